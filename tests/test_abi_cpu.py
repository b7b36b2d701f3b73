"""Host-only checks of the C ABI: the library loads, exports every entry
point the header declares, sizes buffers, and rejects bad arguments with
the documented status before anything is launched (no GPU needed: every
call below fails validation, so no kernel is ever enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_ffn.h")
LIB = os.path.join(ROOT, "activation_sparse_decode_amd", "libsparse_ffn.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsparse_ffn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:sffn|sparse_ffn)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    from activation_sparse_decode_amd import binding
    return binding.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 21, names
    for name in names:
        assert hasattr(L, name), f"{name} declared in sparse_ffn.h but not exported"


def test_sizes(L):
    from activation_sparse_decode_amd import binding as B
    # record = 16-byte header + d_out/2 bytes of codes, rounded to 16 bytes
    assert B.tier_record_bytes(6144, 3) == 16 + 3072
    assert B.tier_record_bytes(4096, 1) == 16 + 2048
    assert B.tier_record_bytes(100, 1) == 80
    assert B.tier_record_bytes(4096, 5) == 0
    assert B.workspace_size(1, 4096, 2048) >= 256 * 2048 * 4
    assert B.workspace_size(16, 17408, 5120) > B.workspace_size(1, 17408, 5120)
    assert L.sffn_abi_version() == 17


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
NULL = None


def status_and_msg(L, rc):
    return rc, L.sffn_last_error().decode()


def select(L, keys=FAKE, key_type=0, rows=1, n=8, ld=8, cluster=1, r_lo=0, r_hi=4, nz=0,
           include=NULL, mask=NULL, ld_mask=0, idx=NULL, ld_idx=0, count=NULL, idx_top=NULL,
           ld_idx_top=0, count_top=NULL, freq=NULL, scale=NULL, exclude=NULL, clear=0):
    return status_and_msg(L, L.sparse_ffn_select(keys, key_type, scale, rows, n, ld, cluster, r_lo,
                                                 r_hi, nz, include, exclude, mask, ld_mask, idx, ld_idx,
                                                 count, idx_top, ld_idx_top, count_top, freq, clear,
                                                 NULL))


def test_select_validation(L):
    rc, msg = select(L, keys=NULL)
    assert rc == 1 and "keys" in msg
    rc, msg = select(L, n=40000, ld=40000)
    assert rc == 2 and "32768" in msg
    rc, msg = select(L, ld=4)
    assert rc == 1 and "ld" in msg
    rc, msg = select(L, r_lo=5)
    assert rc == 1 and "r_lo" in msg
    rc, msg = select(L, key_type=2, nz=1)
    assert rc == 1 and "signed" in msg
    rc, msg = select(L, idx=FAKE, ld_idx=3)
    assert rc == 1 and "ld_idx" in msg
    # with a union mask the index list may hold up to n entries
    rc, msg = select(L, include=FAKE, idx=FAKE, ld_idx=4)
    assert rc == 1 and "ld_idx" in msg
    rc, msg = select(L, key_type=7)
    assert rc == 1 and "key type" in msg
    # clusters: ld must hold n * cluster values
    rc, msg = select(L, cluster=0)
    assert rc == 1 and "cluster" in msg
    rc, msg = select(L, n=8, ld=16, cluster=4)
    assert rc == 1 and "n*cluster" in msg
    rc, msg = select(L, n=5000, ld=10000, cluster=2)
    assert rc == 2 and "4096" in msg
    rc, msg = select(L, n=4096, ld=2**31 - 1, cluster=(1 << 18) + 1)
    assert rc == 2 and "2^30" in msg
    # the top list holds the ranks [0, r_lo)
    rc, msg = select(L, r_lo=3, r_hi=6, idx_top=FAKE, ld_idx_top=2)
    assert rc == 1 and "ld_idx_top" in msg
    # weight-aware keys: fp32 magnitudes of single entries only
    rc, msg = select(L, key_type=1, scale=FAKE)
    assert rc == 1 and "key_scale" in msg
    rc, msg = select(L, n=4, ld=16, cluster=4, scale=FAKE)
    assert rc == 1 and "key_scale" in msg
    rc, msg = select(L, scale=ctypes.c_void_p(0x1002))
    assert rc == 1 and "key_scale" in msg
    rc, msg = select(L, n=4, ld=16, cluster=4, clear=1)
    assert rc == 1 and "clear_keys" in msg
    rc, msg = select(L, scale=FAKE, clear=1)
    assert rc == 1 and "clear_keys" in msg
    rc, msg = select(L, freq=FAKE, clear=1)
    assert rc == 1 and "clear_keys" in msg


def test_row_norms_validation(L):
    rn = L.sparse_ffn_row_norms
    rc, msg = status_and_msg(L, rn(NULL, 8, 64, 64, FAKE, NULL))
    assert rc == 1 and "non-null" in msg
    rc, msg = status_and_msg(L, rn(FAKE, 8, 60, 64, FAKE, NULL))
    assert rc == 1 and "multiple of 8" in msg
    rc, msg = status_and_msg(L, rn(FAKE, 8, 64, 56, FAKE, NULL))
    assert rc == 1 and "ld_w" in msg
    assert status_and_msg(L, rn(FAKE, 0, 64, 64, FAKE, NULL))[0] == 0   # nothing to do


def gemv(L, op=3, W0=FAKE, W1=FAKE, n_rows=64, d=64, ld_w=64, inp=FAKE, batch=1, ld_in=64,
         idx=NULL, count=NULL, k_max=0, group=1, mask=NULL, ld_mask=0, tau=0.0, eps=0.0, aux=NULL,
         ld_aux=0, alpha=NULL, out=FAKE, key=NULL, ld_out=64, acc=0, ws=NULL, ws_bytes=0):
    rc = L.sparse_ffn_gemv(op, W0, W1, n_rows, d, ld_w, inp, batch, ld_in, idx, count, k_max,
                           group, mask, ld_mask, ctypes.c_float(tau), ctypes.c_float(eps), aux, ld_aux, alpha, out, key,
                           ld_out, acc, ws, ws_bytes, NULL)
    return status_and_msg(L, rc)


def test_gemv_validation(L):
    assert gemv(L, op=9)[0] == 1
    rc, msg = gemv(L, op=4, W0=NULL)
    assert rc == 1 and "W0" in msg
    rc, msg = gemv(L, d=12)
    assert rc == 1 and "multiple of 8" in msg
    rc, msg = gemv(L, ld_w=60)
    assert rc == 1 and "ld_w" in msg
    rc, msg = gemv(L, batch=2, d=40, ld_w=40, ld_out=40)
    assert rc == 2 and "d % 32" in msg
    rc, msg = gemv(L, inp=ctypes.c_void_p(0x1004))
    assert rc == 1 and "aligned" in msg
    rc, msg = gemv(L, idx=FAKE, count=NULL, k_max=4)
    assert rc == 1 and "count" in msg
    rc, msg = gemv(L, idx=FAKE, count=FAKE, k_max=3, group=32)
    assert rc == 1 and "exceeds" in msg
    rc, msg = gemv(L)                       # AXPY without a workspace
    assert rc == 3 and "workspace" in msg
    rc, msg = gemv(L, ws=FAKE, ws_bytes=100)
    assert rc == 3
    rc, msg = gemv(L, op=0, W1=NULL, ld_out=64)
    assert rc == 1 and "W1" in msg
    rc, msg = gemv(L, op=1, tau=-1.0, ld_out=64)
    assert rc == 1 and "tau" in msg
    rc, msg = gemv(L, op=2, W0=NULL, aux=NULL, ld_out=64)
    assert rc == 1 and "aux" in msg
    rc, msg = gemv(L, op=0, d=8200, ld_w=8200, ld_in=8200)
    assert rc == 2 and "8192" in msg
    rc, msg = gemv(L, op=0, eps=-1.0)
    assert rc == 1 and "rms_eps" in msg
    rc, msg = gemv(L, op=3, eps=1e-5, ws=FAKE, ws_bytes=1 << 30)
    assert rc == 1 and "rms_eps" in msg
    # thresholded ReGLU and the cluster predictor
    rc, msg = gemv(L, op=5, W1=NULL, ld_out=64)
    assert rc == 1 and "W1" in msg
    rc, msg = gemv(L, op=5, batch=2, ld_out=64)
    assert rc == 2 and "batch 1" in msg
    rc, msg = gemv(L, op=5, tau=-0.5, ld_out=64)
    assert rc == 1 and "tau" in msg
    for theta in (0.0, 1.0, -0.2, 1.5):
        rc, msg = gemv(L, op=6, tau=theta, ld_out=64)
        assert rc == 1 and "probability" in msg, theta
    rc, msg = gemv(L, op=6, tau=0.45, acc=1, ld_out=64)
    assert rc == 1 and "accumulate" in msg
    rc, msg = gemv(L, op=6, tau=0.45, aux=FAKE, ld_aux=10, ld_out=64)
    assert rc == 1 and "bias" in msg
    rc, msg = gemv(L, op=6, tau=0.45, batch=2, ld_out=64)
    assert rc == 2 and "batch 1" in msg
    rc, msg = gemv(L, op=7, idx=FAKE, count=FAKE, k_max=2, group=32, ld_out=64)
    assert rc == 2 and "idx must be NULL" in msg
    rc, msg = gemv(L, op=7, group=48, ld_out=64)
    assert rc == 1 and "dividing" in msg
    rc, msg = gemv(L, op=7, group=32, batch=2, ld_out=64)
    assert rc == 2 and "batch 1" in msg
    rc, msg = gemv(L, op=7, group=32, tau=-1.0, ld_out=64)
    assert rc == 1 and "tau" in msg


def test_gemv_noalloc_limits(L):
    """The allocation-free gemv rejects a product whose scratch exceeds the
    static array before any device work (no GPU needed), and shares
    sparse_ffn_gemv's argument checks."""
    f = L.sparse_ffn_gemv_noalloc
    c = ctypes.c_float
    # batch 1, 64 rows, 16384 outputs: 256 B + 64 KiB per chunk -> within 32 MiB
    # batch 1, d = 2^16: 256 chunks x 256 KiB = 64 MiB -> above it
    rc, msg = status_and_msg(L, f(3, FAKE, NULL, 64, 1 << 16, 1 << 16, FAKE, 1, 64, NULL, NULL, 0,
                                  1, NULL, 0, c(0), c(0), NULL, 0, NULL, FAKE, NULL, 1 << 16, 0,
                                  NULL))
    assert rc == 3 and "static" in msg
    assert L.sparse_ffn_workspace_size(1, 64, 1 << 16) > (32 << 20)
    # batch 256 at d = 5120, 17408 rows: above the array
    assert L.sparse_ffn_workspace_size(256, 17408, 5120) > (32 << 20)
    rc, msg = status_and_msg(L, f(3, FAKE, NULL, 17408, 5120, 5120, FAKE, 256, 17408, NULL, NULL,
                                  0, 1, NULL, 0, c(0), c(0), NULL, 0, NULL, FAKE, NULL, 5120, 0,
                                  NULL))
    assert rc == 3 and "static" in msg
    # the workloads' batched union (batch 16, d = 5120) fits
    assert L.sparse_ffn_workspace_size(16, 17408, 5120) <= (32 << 20)
    # a packed AXPY (op flag 0x100) takes the same scratch and limit
    rc, msg = status_and_msg(L, f(3 | 0x100, FAKE, NULL, 17408, 5120, 5120, FAKE, 256, 17408, NULL,
                                  NULL, 0, 1, NULL, 0, c(0), c(0), NULL, 0, NULL, FAKE, NULL, 5120,
                                  0, NULL))
    assert rc == 3 and "static" in msg
    # row ops take no scratch: their argument errors are sparse_ffn_gemv's
    rc, msg = status_and_msg(L, f(0, FAKE, NULL, 64, 64, 64, FAKE, 1, 64, NULL, NULL, 0, 1, NULL,
                                  0, c(0), c(0), NULL, 0, NULL, FAKE, NULL, 64, 0, NULL))
    assert rc == 1 and "W1" in msg
    rc, msg = status_and_msg(L, f(3, FAKE, NULL, 64, 64, 64, FAKE, 1, 64, FAKE, FAKE, 4, 32, NULL,
                                  0, c(0), c(0), NULL, 0, NULL, FAKE, NULL, 64, 0, NULL))
    assert rc == 1 and "exceeds" in msg


def fused(L, Wg=FAKE, Wu=FAKE, Wd=FAKE, n_rows=64, d=64, ld_w=192, x=FAKE, eps=0.0, idx=NULL,
          count=NULL, k_max=0, a_out=NULL, y=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return status_and_msg(L, L.sparse_ffn_fused_swiglu(Wg, Wu, Wd, n_rows, d, ld_w, x,
                                                       ctypes.c_float(eps), idx, count, k_max,
                                                       a_out, y, 1, ws, ws_bytes, NULL))


def test_fused_swiglu_validation(L):
    """The fused per-neuron SwiGLU entry rejects bad arguments before any
    launch, with the documented status."""
    rc, msg = fused(L, Wd=NULL)
    assert rc == 1 and "Wd" in msg
    rc, msg = fused(L, Wu=ctypes.c_void_p(0x1008))
    assert rc == 1 and "16-byte" in msg
    rc, msg = fused(L, x=NULL)
    assert rc == 1 and "x and y" in msg
    rc, msg = fused(L, d=60, ld_w=192)
    assert rc == 1 and "multiple of 8" in msg
    rc, msg = fused(L, d=4104, ld_w=4104 * 3)
    assert rc == 2 and "4096" in msg
    rc, msg = fused(L, d=64, ld_w=56)
    assert rc == 1 and "ld_w" in msg
    rc, msg = fused(L, eps=-1.0)
    assert rc == 1 and "rms_eps" in msg
    rc, msg = fused(L, eps=float("nan"))
    assert rc == 1 and "rms_eps" in msg
    rc, msg = fused(L, idx=FAKE, count=NULL, k_max=4)
    assert rc == 1 and "count" in msg
    rc, msg = fused(L, idx=FAKE, count=FAKE, k_max=65)
    assert rc == 1 and "k_max" in msg
    rc, msg = fused(L, a_out=ctypes.c_void_p(0x1002))
    assert rc == 1 and "a_out" in msg
    rc, msg = fused(L, ws=NULL, ws_bytes=0)
    assert rc == 3 and "workspace" in msg
    need = L.sparse_ffn_workspace_size(1, 64, 64)
    rc, msg = fused(L, ws_bytes=need - 1)
    assert rc == 3 and "workspace" in msg
    rc, msg = fused(L, ws=ctypes.c_void_p(0x1010))
    assert rc == 1 and "256-byte" in msg


def test_packed_layouts_validation(L):
    """Packed sizes, the pack entry's checks and the gemv flag's limits, all
    rejected before any launch."""
    from activation_sparse_decode_amd import binding as B
    assert L.sparse_ffn_packed_elems(1000, 384, 1) == 1008 * 384      # rows padded to 16
    assert L.sparse_ffn_packed_elems(1000, 512, 2) == 1000 * 512
    assert L.sparse_ffn_packed_elems(1000, 200, 1) == 0               # d % 128
    assert L.sparse_ffn_packed_elems(1000, 384, 2) == 0               # d % 256
    assert L.sparse_ffn_packed_elems(10, 128, 3) == 0
    pk = L.sparse_ffn_pack_weights
    rc, msg = status_and_msg(L, pk(FAKE, 64, 384, 384, 3, ctypes.c_void_p(0x100000), NULL))
    assert rc == 1 and "layout" in msg
    rc, msg = status_and_msg(L, pk(FAKE, 64, 384, 384, 2, ctypes.c_void_p(0x100000), NULL))
    assert rc == 1 and "multiple of 256" in msg
    rc, msg = status_and_msg(L, pk(FAKE, 64, 256, 248, 1, ctypes.c_void_p(0x100000), NULL))
    assert rc == 1 and "ld_w" in msg
    rc, msg = status_and_msg(L, pk(FAKE, 64, 256, 256, 1, ctypes.c_void_p(0x1008), NULL))
    assert rc == 1 and "aligned" in msg
    rc, msg = status_and_msg(L, pk(FAKE, 64, 256, 256, 1, ctypes.c_void_p(0x1000 + 512), NULL))
    assert rc == 1 and "overlaps" in msg
    rc, msg = status_and_msg(L, pk(NULL, 64, 256, 256, 1, FAKE, NULL))
    assert rc == 1 and "non-null" in msg
    # the gemv flag: batched kernels only, ld_w == d, the layout's d multiple
    rc, msg = gemv(L, op=B.OP_GLU_SILU | B.PACKED, ld_out=64)
    assert rc == 2 and "batch > 1" in msg
    rc, msg = gemv(L, op=B.OP_GLU_SILU | B.PACKED, d=256, ld_w=264, batch=4, ld_out=64, ld_in=256)
    assert rc == 1 and "ld_w == d" in msg
    rc, msg = gemv(L, op=B.OP_GLU_SILU | B.PACKED, d=96, ld_w=96, batch=4, ld_out=64, ld_in=96)
    assert rc == 2 and "128" in msg
    rc, msg = gemv(L, op=B.OP_AXPY | B.PACKED, d=384, ld_w=384, batch=4, ld_out=384, ld_in=64)
    assert rc == 2 and "256" in msg
    rc, msg = gemv(L, op=B.OP_GLU_RELU | B.PACKED, d=256, ld_w=256, batch=4, ld_out=64, ld_in=256)
    assert rc == 2 and "batch 1" in msg


def test_masked_rows_validation(L):
    """SFFN_MASKED_ROWS: AXPY only, batch > 1, no index list, a 16-byte
    aligned mask with a row stride of a multiple of 16; rejected before any
    launch."""
    from activation_sparse_decode_amd import binding as B
    op = B.OP_AXPY | B.MASKED_ROWS
    kw = dict(n_rows=64, d=256, ld_w=256, batch=4, ld_in=64, ld_out=256, ws=FAKE, ws_bytes=1 << 30)
    rc, msg = gemv(L, op=op, **{**kw, "batch": 1})
    assert rc == 2 and "batch > 1" in msg
    rc, msg = gemv(L, op=op, **kw)
    assert rc == 1 and "row_mask" in msg
    rc, msg = gemv(L, op=op, idx=FAKE, count=FAKE, k_max=4, mask=FAKE, ld_mask=64, **kw)
    assert rc == 1 and "idx must be NULL" in msg
    rc, msg = gemv(L, op=op, mask=FAKE, ld_mask=72, **kw)
    assert rc == 1 and "ld_mask" in msg
    rc, msg = gemv(L, op=op, mask=ctypes.c_void_p(0x1004), ld_mask=64, **kw)
    assert rc == 1 and "aligned" in msg
    rc, msg = gemv(L, op=B.OP_GLU_SILU | B.MASKED_ROWS, mask=FAKE, ld_mask=64,
                   **{**kw, "ld_in": 256, "ld_out": 64})
    assert rc == 1 and "AXPY only" in msg


def gemv_lists(L, n=2, W=(FAKE, FAKE), n_rows=(64, 64), d=64, ld_w=64, inp=(FAKE, FAKE),
               idx=(FAKE, FAKE), count=(FAKE, FAKE), k_max=(2, 2), group=32, alpha=None, out=FAKE,
               ws=FAKE, ws_bytes=1 << 30, null_arrays=False):
    P = ctypes.c_void_p
    I = ctypes.c_int
    arr = lambda T, vs: (T * len(vs))(*vs)  # noqa: E731
    rc = L.sparse_ffn_gemv_lists(
        n, None if null_arrays else arr(P, W), arr(I, n_rows), d, ld_w, arr(P, inp), arr(P, idx),
        arr(P, count), arr(I, k_max), group, None if alpha is None else arr(P, alpha), out, 1, ws,
        ws_bytes, NULL)
    return status_and_msg(L, rc)


def test_gemv_lists_validation(L):
    rc, msg = gemv_lists(L, n=0)
    assert rc == 1 and "n_lists" in msg
    rc, msg = gemv_lists(L, n=9)
    assert rc == 1 and "n_lists" in msg
    rc, msg = gemv_lists(L, null_arrays=True)
    assert rc == 1 and "host arrays" in msg
    rc, msg = gemv_lists(L, W=(FAKE, NULL))
    assert rc == 1 and "W[1]" in msg
    rc, msg = gemv_lists(L, idx=(FAKE, NULL))
    assert rc == 1 and "idx[1]" in msg
    rc, msg = gemv_lists(L, k_max=(2, 3))       # 3 clusters of 32 rows > 64 rows
    assert rc == 1 and "exceeds" in msg
    rc, msg = gemv_lists(L, d=60, ld_w=64)
    assert rc == 1 and "multiple of 8" in msg
    rc, msg = gemv_lists(L, group=0)
    assert rc == 1 and "group" in msg
    rc, msg = gemv_lists(L, alpha=(FAKE, ctypes.c_void_p(0x1002)))
    assert rc == 1 and "alpha[1]" in msg
    rc, msg = gemv_lists(L, ws=NULL, ws_bytes=0)
    assert rc == 3 and "workspace" in msg
    rc, msg = gemv_lists(L, ws_bytes=64)
    assert rc == 3


def test_score_validation(L):
    sc = L.sparse_ffn_score
    assert status_and_msg(L, sc(5, FAKE, 1, 8, 8, 1, 0, NULL, 0, FAKE, NULL))[0] == 1
    rc, msg = status_and_msg(L, sc(1, FAKE, 1, 100, 100, 32, 0, NULL, 0, FAKE, NULL))
    assert rc == 1 and "multiple" in msg
    rc, msg = status_and_msg(L, sc(2, FAKE, 1, 8, 8, 1, 0, NULL, 2, FAKE, NULL))
    assert rc == 1 and "picked" in msg
    rc, msg = status_and_msg(L, sc(0, FAKE, 1, 8, 4, 1, 0, NULL, 0, FAKE, NULL))
    assert rc == 1 and "ld" in msg


def test_tier_validation(L):
    seg = (ctypes.c_int32 * 4)(0, 4096, 5120, 6144)
    bad = (ctypes.c_int32 * 4)(0, 4000, 5120, 6144)
    enc = L.sparse_ffn_encode_tiers
    rc, msg = status_and_msg(L, enc(FAKE, 6144, 16, 6144, bad, 3, FAKE, 3088, NULL))
    assert rc == 1 and "multiple of 64" in msg
    rc, msg = status_and_msg(L, enc(FAKE, 6144, 16, 6144, seg, 3, FAKE, 3072, NULL))
    assert rc == 1 and "rec_bytes" in msg
    rc, msg = status_and_msg(L, enc(FAKE, 6144, 16, 6144, seg, 5, FAKE, 3088, NULL))
    assert rc == 2
    tg = L.sparse_ffn_tiered_gemv
    rc, msg = status_and_msg(L, tg(FAKE, 6144, FAKE, 3088, seg, 3, 4096, 6144, FAKE, FAKE, FAKE, 614,
                                   NULL, NULL, 1433, FAKE, 0, FAKE, 1 << 30, NULL))
    assert rc == 1 and "mid list" in msg
    rc, msg = status_and_msg(L, tg(FAKE, 6144, FAKE, 3088, seg, 3, 4096, 6144, FAKE, FAKE, FAKE, 614,
                                   FAKE, FAKE, 1433, FAKE, 0, FAKE, 64, NULL))
    assert rc == 3 and "workspace" in msg
    tk = L.sparse_ffn_tiered_gemv_keyed
    thr = ctypes.c_void_p(0x1008)

    def keyed(n_in=4096, keys=FAKE, key_type=0, thr_top=thr, thr=thr, k_top=614, k_mid=1433,
              x=FAKE, ws_bytes=1 << 30, seg_=seg, n_seg=3):
        return status_and_msg(L, tk(FAKE, 6144, FAKE, 3088, seg_, n_seg, n_in, 6144, x, keys,
                                    key_type, thr_top, thr, k_top, k_mid, FAKE, 0, FAKE, ws_bytes,
                                    NULL))

    rc, msg = keyed(x=NULL)
    assert rc == 1 and "non-null" in msg
    rc, msg = keyed(n_in=600000, k_top=10, k_mid=10)
    assert rc == 2 and "524288" in msg
    rc, msg = keyed(keys=NULL)
    assert rc == 1 and "keys" in msg
    rc, msg = keyed(key_type=3)
    assert rc == 1 and "key type" in msg
    rc, msg = keyed(thr_top=NULL)
    assert rc == 1 and "thr_top" in msg
    rc, msg = keyed(thr=ctypes.c_void_p(0x1004))
    assert rc == 1 and "8-byte" in msg
    rc, msg = keyed(k_mid=5000)
    assert rc == 1 and "k_mid_max" in msg
    rc, msg = keyed(n_seg=5)
    assert rc == 2
    rc, msg = keyed(ws_bytes=64)
    assert rc == 3 and "workspace" in msg


def test_compact_validation(L):
    cp = L.sparse_ffn_compact
    rc, msg = status_and_msg(L, cp(FAKE, 100, 64, 64, FAKE, 101, 0, FAKE, 64, NULL))
    assert rc == 1 and "k=" in msg
    rc, msg = status_and_msg(L, cp(FAKE, 100, 64, 64, FAKE, 10, 0, FAKE, 60, NULL))
    assert rc == 1 and "ld_out" in msg
    rc, msg = status_and_msg(L, cp(FAKE, 100, 64, 64, FAKE, 10, 1, FAKE, 4, NULL))
    assert rc == 1 and "ld_out" in msg
    rc, msg = status_and_msg(L, cp(FAKE, 100, 64, 64, NULL, 10, 1, FAKE, 16, NULL))
    assert rc == 1 and "idx" in msg


def rowop_lists(L, op=0, n=2, W0=(FAKE, FAKE), W1=(FAKE, FAKE), n_rows=64, d=64, ld_w=64, x=FAKE,
                idx=None, count=(FAKE, FAKE), k_max=(2, 2), group=1, tau=0.0, eps=0.0, aux=None,
                out=(FAKE, FAKE), key=None, acc=0):
    P, I = ctypes.c_void_p, ctypes.c_int
    arr = lambda T, vs: None if vs is None else (T * len(vs))(*vs)  # noqa: E731
    rc = L.sparse_ffn_rowop_lists(op, n, arr(P, W0), arr(P, W1), n_rows, d, ld_w, x, arr(P, idx),
                                  arr(P, count), arr(I, k_max), group, ctypes.c_float(tau),
                                  ctypes.c_float(eps), arr(P, aux), arr(P, out), arr(P, key), acc,
                                  NULL)
    return status_and_msg(L, rc)


def test_rowop_lists_validation(L):
    rc, msg = rowop_lists(L, op=3)
    assert rc == 1 and "not a row op" in msg
    rc, msg = rowop_lists(L, n=0)
    assert rc == 1 and "n_lists" in msg
    rc, msg = rowop_lists(L, n=9)
    assert rc == 1 and "n_lists" in msg
    rc, msg = rowop_lists(L, out=None)
    assert rc == 1 and "out" in msg
    rc, msg = rowop_lists(L, d=5128, ld_w=5128)
    assert rc == 2 and "5120" in msg
    rc, msg = rowop_lists(L, W1=None)
    assert rc == 1 and "W1" in msg
    rc, msg = rowop_lists(L, op=2, W0=None, aux=None)
    assert rc == 1 and "aux" in msg
    rc, msg = rowop_lists(L, idx=(FAKE, FAKE), k_max=None)
    assert rc == 1 and "k_max" in msg
    rc, msg = rowop_lists(L, idx=(FAKE, FAKE), k_max=(2, 65))
    assert rc == 1 and "exceeds" in msg
    rc, msg = rowop_lists(L, W0=(FAKE, ctypes.c_void_p(0x1008)))
    assert rc == 1 and "W0[1]" in msg
    rc, msg = rowop_lists(L, op=6, tau=1.0)
    assert rc == 1 and "probability" in msg
    rc, msg = rowop_lists(L, op=6, tau=0.45, acc=1)
    assert rc == 1 and "accumulate" in msg
    rc, msg = rowop_lists(L, op=5, tau=-1.0)
    assert rc == 1 and "tau" in msg
    rc, msg = rowop_lists(L, x=ctypes.c_void_p(0x1004))
    assert rc == 1 and "x must" in msg
    rc, msg = rowop_lists(L, op=7, idx=(FAKE, FAKE), group=32)
    assert rc == 2 and "idx NULL" in msg
    rc, msg = rowop_lists(L, op=7, group=48)
    assert rc == 1 and "dividing" in msg


def test_gather_validation(L):
    g = L.sparse_ffn_gather
    rc, msg = status_and_msg(L, g(FAKE, 0, FAKE, NULL, 4, FAKE, NULL))
    assert rc == 1 and "n_src" in msg
    rc, msg = status_and_msg(L, g(FAKE, 10, FAKE, NULL, -1, FAKE, NULL))
    assert rc == 1 and "k_max" in msg
    rc, msg = status_and_msg(L, g(FAKE, 10, NULL, NULL, 4, FAKE, NULL))
    assert rc == 1 and "non-null" in msg
    rc, msg = status_and_msg(L, g(FAKE, 10, FAKE, ctypes.c_void_p(0x1002), 4, FAKE, NULL))
    assert rc == 1 and "aligned" in msg
    assert g(FAKE, 10, NULL, NULL, 0, FAKE, NULL) == 0     # nothing to gather: no launch


def test_select_threshold_validation(L):
    t = L.sparse_ffn_select_threshold
    ok_thr = ctypes.c_void_p(0x1008)

    def call(keys=FAKE, key_type=1, rows=1, n=8, ld=8, k=4, thr=ok_thr, k_top=0, thr_top=NULL):
        return status_and_msg(L, t(keys, key_type, rows, n, ld, k_top, k, thr_top, thr, NULL))

    rc, msg = call(keys=NULL)
    assert rc == 1 and "keys" in msg
    rc, msg = call(key_type=3)
    assert rc == 1 and "key type" in msg
    rc, msg = call(rows=-1)
    assert rc == 1 and "rows" in msg
    rc, msg = call(n=40000, ld=40000)
    assert rc == 2 and "32768" in msg
    rc, msg = call(ld=4)
    assert rc == 1 and "ld" in msg
    rc, msg = call(k=-1)
    assert rc == 1 and "k=" in msg
    rc, msg = call(keys=ctypes.c_void_p(0x1002))
    assert rc == 1 and "4-byte" in msg
    rc, msg = call(thr=NULL)
    assert rc == 1 and "thr_out" in msg
    rc, msg = call(thr=ctypes.c_void_p(0x1004))
    assert rc == 1 and "8-byte" in msg
    rc, msg = call(k_top=5, thr_top=ok_thr)
    assert rc == 1 and "k_top=5" in msg
    rc, msg = call(k_top=-1, thr_top=ok_thr)
    assert rc == 1 and "k_top=-1" in msg
    rc, msg = call(k_top=2)
    assert rc == 1 and "needs thr_top_out" in msg
    rc, msg = call(k_top=2, thr_top=ctypes.c_void_p(0x1004))
    assert rc == 1 and "thr_top_out" in msg and "8-byte" in msg
    assert call(rows=0)[0] == 0                            # nothing to select: no launch


def test_gemv_keyed_validation(L):
    g = L.sparse_ffn_gemv_keyed
    ws_ok = ctypes.c_void_p(0x100000)
    big = 1 << 30

    def call(W=FAKE, n_rows=64, d=256, ld_w=256, inp=FAKE, keys=FAKE, key_type=1,
             thr=ctypes.c_void_p(0x1008), k_max=32, alpha=NULL, out=FAKE, acc=0, ws=ws_ok,
             ws_bytes=big):
        return status_and_msg(L, g(W, n_rows, d, ld_w, inp, keys, key_type, thr, k_max, alpha,
                                   out, acc, ws, ws_bytes, NULL))

    rc, msg = call(W=NULL)
    assert rc == 1 and "W must" in msg
    rc, msg = call(W=ctypes.c_void_p(0x1008))
    assert rc == 1 and "W must" in msg
    rc, msg = call(inp=NULL)
    assert rc == 1 and "in must" in msg
    rc, msg = call(out=ctypes.c_void_p(0x1004))
    assert rc == 1 and "out must" in msg
    rc, msg = call(keys=NULL)
    assert rc == 1 and "keys" in msg
    rc, msg = call(key_type=5)
    assert rc == 1 and "key type" in msg
    rc, msg = call(thr=ctypes.c_void_p(0x1004))
    assert rc == 1 and "thr" in msg
    rc, msg = call(n_rows=0)
    assert rc == 1 and "n_rows" in msg
    rc, msg = call(d=100, ld_w=104)
    assert rc == 1 and "d=100" in msg
    rc, msg = call(ld_w=200)
    assert rc == 1 and "ld_w" in msg
    rc, msg = call(k_max=65)
    assert rc == 1 and "k_max" in msg
    rc, msg = call(alpha=ctypes.c_void_p(0x1002))
    assert rc == 1 and "alpha" in msg
    rc, msg = call(n_rows=270000, k_max=10)
    assert rc == 2 and "chunks" in msg
    rc, msg = call(ws=NULL)
    assert rc == 3 and "workspace" in msg
    rc, msg = call(ws_bytes=100)
    assert rc == 3 and "workspace" in msg
    rc, msg = call(ws=ctypes.c_void_p(0x100010))
    assert rc == 1 and "256-byte" in msg


def test_no_fallback_when_library_missing(monkeypatch):
    from activation_sparse_decode_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", "/nonexistent/libsparse_ffn.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        binding.lib()
