"""The batched AXPY with SFFN_MASKED_ROWS: no index list, the union of the
tokens' masks formed inside the product.  Against the oracle over each
token's own rows, and bitwise against itself with every row outside the
union NaN-poisoned (those rows are never read), row-major and packed.
Shapes: a ragged row count (mask rows padded to 16 bytes), the 17408 x 5120
layer at batch 4 / 16 / 19 (two token tiles), and 140000 narrow rows, whose
chunks span more than one 2048-row segment, with a long stretch that no
token selects (segments with no live row)."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from gpu_common import assert_close, banner, dev, gpu, host, needs_gpu

pytestmark = [gpu, needs_gpu]

NAN_BF16 = np.uint16(0x7FC0)


def masks(rng, batch, N, frac, dead=None):
    M = (rng.random((batch, N)) < frac).astype(np.uint8)
    if dead is not None:
        M[:, dead[0]:dead[1]] = 0
    return M


def run(WdT, A, M, packed, ws):
    batch, N = A.shape
    d = WdT.shape[1]
    W = dev(WdT)
    if packed:
        W = B.pack_weights(W, B.LAYOUT_COL_PANELS)
    ldm = (N + 15) // 16 * 16
    Md = torch.zeros(batch, ldm, dtype=torch.uint8, device="cuda")
    Md[:, :N] = dev(M)
    Y = torch.full((batch, d), 0.5, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_AXPY | B.MASKED_ROWS, W, None, dev(A), Y, row_mask=Md[:, :N],
                      accumulate=True, workspace=ws)
    torch.cuda.synchronize()
    return host(Y)


@pytest.mark.parametrize("batch,N,d,frac,dead", [
    (4, 1000, 256, 0.3, None),
    (4, 17408, 5120, 0.4, None),
    (16, 17408, 5120, 0.4, None),
    (19, 17408, 5120, 0.4, (3000, 9000)),
    (16, 140000, 256, 0.05, (20000, 60000)),
])
def test_masked_rows(batch, N, d, frac, dead):
    banner(f"masked rows batch={batch} N={N} d={d}")
    WdT = synth.weight_bf16(batch, synth.W_C4, 5, 0, synth.T_DOWN, N, d)
    rng = np.random.default_rng(N + batch)
    A = rng.standard_normal((batch, N)).astype(np.float32)
    M = masks(rng, batch, N, frac, dead)
    U = np.flatnonzero(M.any(axis=0))
    ws = B.new_workspace(batch, N, d)
    P = np.full_like(WdT, NAN_BF16)
    P[U] = WdT[U]
    for packed in ((False, True) if d % 256 == 0 else (False,)):
        y = run(WdT, A, M, packed, ws)
        for b in sorted({0, batch // 2, batch - 1}):
            s = np.flatnonzero(M[b])
            assert_close(y[b] - 0.5, oracle.down_gather(WdT, s, A[b][s]),
                         what=f"token {b} packed={packed}")
        yp = run(P, A, M, packed, ws)
        assert np.all(np.isfinite(yp)), "a row outside the union (NaN) was read"
        assert np.array_equal(yp.view(np.uint32), y.view(np.uint32))
        # run to run: the same bits
        assert np.array_equal(run(WdT, A, M, packed, ws).view(np.uint32), y.view(np.uint32))


def test_masked_rows_arguments():
    """The flag's requirements, rejected before any launch."""
    banner("masked rows arguments")
    W = torch.zeros(64, 256, dtype=torch.int16, device="cuda")
    A = torch.zeros(4, 64, dtype=torch.float32, device="cuda")
    Y = torch.zeros(4, 256, dtype=torch.float32, device="cuda")
    ws = B.new_workspace(4, 64, 256)
    M = torch.zeros(4, 64, dtype=torch.uint8, device="cuda")
    cases = [
        (dict(op=B.OP_AXPY | B.MASKED_ROWS, row_mask=None), B.SFFN_EINVAL),
        (dict(op=B.OP_AXPY | B.MASKED_ROWS, row_mask=M, idx=torch.zeros(4, dtype=torch.int32,
                                                                        device="cuda"),
              count=torch.zeros(1, dtype=torch.int32, device="cuda"), k_max=4), B.SFFN_EINVAL),
        (dict(op=B.OP_AXPY | B.MASKED_ROWS, row_mask=torch.zeros(4, 72, dtype=torch.uint8,
                                                                 device="cuda")[:, :64]),
         B.SFFN_EINVAL),
        (dict(op=B.OP_GLU_SILU | B.MASKED_ROWS, row_mask=M), B.SFFN_EINVAL),
    ]
    for kw, status in cases:
        op = kw.pop("op")
        with pytest.raises(B.SffnError) as e:
            if op & 0xFF == B.OP_GLU_SILU:
                B.sparse_ffn_gemv(op, W, W, torch.zeros(4, 256, device="cuda"),
                                  torch.zeros(4, 64, device="cuda"), **kw)
            else:
                B.sparse_ffn_gemv(op, W, None, A, Y, workspace=ws, **kw)
        assert e.value.status == status, (kw, e.value)
    with pytest.raises(B.SffnError) as e:
        B.sparse_ffn_gemv(B.OP_AXPY | B.MASKED_ROWS, W, None, A[0], Y[0], row_mask=M[0],
                          workspace=B.new_workspace(1, 64, 256))
    assert e.value.status == B.SFFN_EUNSUPPORTED
