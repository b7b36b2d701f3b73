"""SpAx three-tier read (Llama3.1-8B QKV and down at full size): the 4-bit
encoder is bit-exact with the oracle's, the tiers are bit-exact rank
ranges of |x| (as index lists, or as threshold pairs the product reads the
keys with), and the product is within tolerance of the oracle's."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import TieredProjection, pct_count, threshold_members
from gpu_common import assert_close, banner, dev, gpu, host, needs_gpu

pytestmark = [gpu, needs_gpu]

CASES = {
    "small": (512, 384, [0, 256, 320, 384]),
    "qkv": (4096, 6144, [0, 4096, 5120, 6144]),
    "down": (14336, 4096, [0, 4096]),
}


def make(name, seed=0):
    n_in, n_out, seg = CASES[name]
    t = synth.T_QKV if name != "down" else synth.T_DOWN
    Wt = synth.weight_bf16(seed, synth.W_C2, 0, 0, t, n_in, n_out)
    x = synth.tokens(seed, synth.W_C2, 1 + len(name), 1, n_in)[0]
    return Wt, x, seg


def unpack_records(rec: np.ndarray, n_out: int, n_seg: int):
    hdr = rec[:, :16].copy().view(np.uint16)            # [n_in][8]
    scale = hdr[:, 0:2 * n_seg:2].view(np.float16)
    zero = hdr[:, 1:2 * n_seg:2].view(np.float16)
    codes = rec[:, 16:16 + n_out // 2]
    q = np.empty((rec.shape[0], n_out), dtype=np.uint8)
    q[:, 0::2] = codes & 0x0F
    q[:, 1::2] = codes >> 4
    return scale, zero, q


@pytest.mark.parametrize("keyed", [True, False])
@pytest.mark.parametrize("name", ["small", "qkv", "down"])
def test_tiered_stagewise(name, keyed):
    banner(f"c2 {name} keyed={keyed}")
    Wt, x, seg = make(name)
    n_in, n_out = Wt.shape
    k_top, k_mid = pct_count(15, n_in), pct_count(35, n_in)
    proj = TieredProjection(dev(Wt), seg, k_top, k_mid, keyed=keyed)
    y = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    xd = dev(x)
    proj(xd, y)
    torch.cuda.synchronize()
    scale, zero, q = unpack_records(host(proj.rec), n_out, len(seg) - 1)
    o_scale, o_zero, o_q = oracle.encode_4bit(Wt, seg)
    assert np.array_equal(scale.view(np.uint16), o_scale.view(np.uint16))
    assert np.array_equal(zero.view(np.uint16), o_zero.view(np.uint16))
    assert np.array_equal(q, o_q)
    top, mid = proj.tiers(xd)
    o_top, o_mid = oracle.tier_sets(x, k_top, k_mid)
    assert np.array_equal(top, o_top) and np.array_equal(mid, o_mid)
    y_ref = oracle.tiered_gemv(Wt, o_scale, o_zero, o_q, seg, x, top, mid)
    e = assert_close(host(y), y_ref, what="tiered product")
    dense = oracle.widen_bf16(Wt).T @ x.astype(np.float64)
    print(f"  err {e:.2e}; vs dense product {np.max(np.abs(host(y) - dense)) / np.sqrt(np.mean(dense**2)):.3f} (approximation, reported)")

    # skipped columns are never read: poison their weights and records
    skipped = np.setdiff1d(np.arange(n_in), np.concatenate([top, mid]))
    Wp = Wt.copy()
    Wp[skipped] = 0x7FC0
    Wp[mid] = 0x7FC0                       # middle tier reads codes only
    rec = host(proj.rec).copy()
    rec[skipped] = 0xFF
    rec[skipped, :16] = np.frombuffer(np.array([0x7E00] * 8, np.uint16).tobytes(), np.uint8)
    rec[top] = 0xFF
    y2 = torch.zeros_like(y)
    if keyed:
        B.sparse_ffn_tiered_gemv_keyed(dev(Wp), dev(rec), seg, xd, xd, B.KEY_ABS_F32, proj.thr[0],
                                       proj.thr[1], k_top, k_mid, y2, workspace=proj.ws)
    else:
        B.sparse_ffn_tiered_gemv(dev(Wp), dev(rec), seg, xd, proj.idx_top, proj.cnt[0:1], k_top,
                                 proj.idx_mid, proj.cnt[1:2], k_mid, y2, workspace=proj.ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))


def test_keyed_tiers_with_ties():
    """Both tier bounds inside runs of equal |x| (index order decides), and
    the product over those tiers; several (k_top, k_mid) splits, including an
    empty top or middle tier and everything selected."""
    banner("c2 keyed ties")
    n_in, n_out, seg = CASES["qkv"]
    Wt = synth.weight_bf16(11, synth.W_C2, 0, 0, synth.T_QKV, n_in, n_out)
    rng = np.random.default_rng(11)
    x = (rng.integers(0, 6, n_in) * rng.choice([-1, 1], n_in)).astype(np.float32) * 0.25
    xd = dev(x)
    o_scale, o_zero, o_q = oracle.encode_4bit(Wt, seg)
    y = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    proj = TieredProjection(dev(Wt), seg, 1, 1)
    for k_top, k_mid in [(700, 1300), (0, 2000), (1500, 0), (1, n_in - 1), (n_in, 0)]:
        thr = torch.zeros(2, 2, dtype=torch.int32, device="cuda")
        B.sparse_ffn_select_threshold(xd, B.KEY_ABS_F32, k_top + k_mid, thr[1], k_top=k_top,
                                      thr_top_out=thr[0])
        ws = B.new_workspace(1, k_top + k_mid, n_out)
        B.sparse_ffn_tiered_gemv_keyed(proj.Wt, proj.rec, seg, xd, xd, B.KEY_ABS_F32, thr[0],
                                       thr[1], k_top, k_mid, y, workspace=ws)
        torch.cuda.synchronize()
        key = x.view(np.uint32) & np.uint32(0x7FFFFFFF)
        T = host(thr)
        top = threshold_members(key, T[0])
        mid = np.setdiff1d(threshold_members(key, T[1]), top)
        o_top, o_mid = oracle.tier_sets(x, k_top, k_mid)
        assert np.array_equal(top, o_top) and np.array_equal(mid, o_mid), (k_top, k_mid)
        y_ref = oracle.tiered_gemv(Wt, o_scale, o_zero, o_q, seg, x, o_top, o_mid)
        if o_top.size + o_mid.size:
            assert_close(host(y), y_ref, what=f"keyed ties {k_top}/{k_mid}")


def test_keyed_tiers_accumulate_graph_replay():
    """The threshold select (both pairs) and the keyed tiered product with
    accumulate, captured in a HIP graph: every replay on new inputs gives
    the eager bits, and the eager result is y0 plus the oracle's product."""
    banner("c2 keyed accumulate + graph replay")
    n_in, n_out, seg = CASES["qkv"]
    Wt = synth.weight_bf16(13, synth.W_C2, 0, 0, synth.T_QKV, n_in, n_out)
    xs = [synth.tokens(13, synth.W_C2, 20 + i, 1, n_in)[0] for i in range(3)]
    y0 = np.random.default_rng(13).standard_normal(n_out).astype(np.float32)
    k_top, k_mid = pct_count(15, n_in), pct_count(35, n_in)
    proj = TieredProjection(dev(Wt), seg, k_top, k_mid)
    x = torch.zeros(n_in, dtype=torch.float32, device="cuda")
    y = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    y0d = dev(y0)

    def body():
        B.sparse_ffn_select_threshold(x, B.KEY_ABS_F32, k_top + k_mid, proj.thr[1], k_top=k_top,
                                      thr_top_out=proj.thr[0])
        B.sparse_ffn_tiered_gemv_keyed(proj.Wt, proj.rec, seg, x, x, B.KEY_ABS_F32, proj.thr[0],
                                       proj.thr[1], k_top, k_mid, y, accumulate=True,
                                       workspace=proj.ws)

    o_scale, o_zero, o_q = oracle.encode_4bit(Wt, seg)
    eager = []
    for v in xs:
        x.copy_(torch.from_numpy(v).cuda())
        y.copy_(y0d)
        body()
        torch.cuda.synchronize()
        eager.append(host(y).copy())
        top, mid = oracle.tier_sets(v, k_top, k_mid)
        ref = y0.astype(np.float64) + oracle.tiered_gemv(Wt, o_scale, o_zero, o_q, seg, v, top, mid)
        assert_close(eager[-1], ref, what="keyed tiers, accumulate")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    torch.cuda.synchronize()
    for rep in range(2):
        for v, ref in zip(xs, eager):
            x.copy_(torch.from_numpy(v).cuda())
            y.copy_(y0d)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host(y).view(np.uint32), ref.view(np.uint32)), rep


@pytest.mark.parametrize("n_in", [40000, 131072, 524288])
def test_keyed_tiers_many_chunks(n_in):
    """Inputs past the select's row limit (pairs built on the host from the
    oracle's order): tier chunks of one to four passes of 1024 inputs, up to
    the largest input count."""
    banner(f"c2 keyed n_in={n_in}")
    n_out, seg = (128, [0, 64, 128]) if n_in < 500000 else (64, [0, 64])
    Wt = synth.weight_bf16(12, synth.W_C2, 0, 0, synth.T_DOWN, n_in, n_out)
    x = synth.tokens(12, synth.W_C2, 9, 1, n_in)[0]
    k_top, k_mid = pct_count(10, n_in), pct_count(30, n_in)
    proj = TieredProjection(dev(Wt), seg, k_top, k_mid)
    key = x.view(np.uint32) & np.uint32(0x7FFFFFFF)
    order = oracle.rank_order(key)

    def pair(k):
        if k == 0:
            return [0xFFFFFFFF, 0xFFFFFFFF]
        e = int(order[k - 1])
        return [int(key[e]), e]

    thr = dev(np.array([pair(k_top), pair(k_top + k_mid)], dtype=np.int64).astype(np.uint32))
    y = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    xd = dev(x)
    B.sparse_ffn_tiered_gemv_keyed(proj.Wt, proj.rec, seg, xd, xd, B.KEY_ABS_F32, thr[0], thr[1],
                                   k_top, k_mid, y, workspace=proj.ws)
    torch.cuda.synchronize()
    o_top, o_mid = oracle.tier_sets(x, k_top, k_mid)
    assert np.array_equal(threshold_members(key, host(thr)[0]), o_top)
    o_scale, o_zero, o_q = oracle.encode_4bit(Wt, seg)
    y_ref = oracle.tiered_gemv(Wt, o_scale, o_zero, o_q, seg, x, o_top, o_mid)
    assert_close(host(y), y_ref, what=f"keyed n_in={n_in}")


def test_tier_special_cases():
    banner("c2 special cases")
    Wt, x, seg = make("small", seed=3)
    n_in, n_out = Wt.shape
    xd = dev(x)
    # all columns in the top tier: the dense product
    proj = TieredProjection(dev(Wt), seg, n_in, 0)
    y = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    proj(xd, y)
    torch.cuda.synchronize()
    assert_close(host(y), oracle.widen_bf16(Wt).T @ x.astype(np.float64), what="all top")
    # k_mid = 0: the gathered product of the top columns
    proj = TieredProjection(dev(Wt), seg, 100, 0)
    proj(xd, y)
    torch.cuda.synchronize()
    top = oracle.tier_sets(x, 100, 0)[0]
    assert_close(host(y), oracle.down_gather(Wt, top, x[top]), what="top only")
    # weights on a 4-bit grid: the middle tier reproduces them exactly
    rng = np.random.default_rng(4)
    grid = np.zeros((n_in, n_out), np.float32)
    for s in range(len(seg) - 1):
        lo, hi = seg[s], seg[s + 1]
        qq = rng.integers(0, 16, size=(n_in, hi - lo))
        qq[:, 0], qq[:, 1] = 0, 15
        grid[:, lo:hi] = -0.5 + 0.0625 * qq
    Wg = synth.f32_to_bf16_bits(grid)
    proj = TieredProjection(dev(Wg), seg, 0, n_in)
    proj(xd, y)
    torch.cuda.synchronize()
    assert_close(host(y), grid.T.astype(np.float64) @ x.astype(np.float64), tol=1e-5, what="grid")
    # empty tiers: y = 0
    proj = TieredProjection(dev(Wt), seg, 0, 0)
    y.fill_(5.0)
    proj(xd, y)
    torch.cuda.synchronize()
    assert np.all(host(y) == 0.0)


# ------------------------------------------------------------------ WiSparse weight-aware tiers
@pytest.mark.parametrize("n_rows,d", [(1, 8), (7, 520), (4096, 6144), (14336, 4096)])
def test_row_norms(n_rows, d):
    """||W^T[j]||_2 per row: fp32 accumulation within 1e-5 relative of the
    oracle's fp64 (about sqrt(d/8) rounding steps per lane plus the 64-lane
    tree, far below the bound), and bit-exact where the sum of squares is an
    integer below 2^24 (exact in any order; the fp32 square root is correctly
    rounded, as is the fp64 one rounded to fp32)."""
    banner(f"row norms {n_rows}x{d}")
    Wt = synth.weight_bf16(5, synth.W_C2, 0, 0, synth.T_DOWN, n_rows, d)
    out = torch.full((n_rows,), -1.0, dtype=torch.float32, device="cuda")
    B.sparse_ffn_row_norms(dev(Wt), out)
    torch.cuda.synchronize()
    ref = oracle.row_norms(Wt)
    np.testing.assert_allclose(host(out), ref, rtol=1e-5, atol=0)
    rng = np.random.default_rng(n_rows + d)
    Wi = rng.integers(-8, 9, size=(n_rows, d)).astype(np.float32)
    Wi[0] = 0.0                                            # a zero row
    B.sparse_ffn_row_norms(dev(synth.f32_to_bf16_bits(Wi)), out)
    torch.cuda.synchronize()
    exp = oracle.row_norms(synth.f32_to_bf16_bits(Wi)).astype(np.float32)
    assert np.array_equal(host(out).view(np.uint32), exp.view(np.uint32))
    # a row stride wider than the row
    Wp = np.zeros((n_rows, d + 64), np.uint16)
    Wp[:, :d] = Wt
    Wp[:, d:] = 0x7FC0                                     # never read
    B.sparse_ffn_row_norms(dev(Wp)[:, :d], out)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(out), ref, rtol=1e-5, atol=0)


@pytest.mark.parametrize("name", ["small", "qkv", "down"])
def test_weight_aware_tiers(name):
    """Tiers ranked by |x_j| * ||W[:, j]||_2.  With integer weights the GPU
    norms equal the oracle's, so the tiers are bit-exact end to end; with the
    workload's weights the norms agree to rounding (checked on their own) and
    the tiers are bit-exact with the oracle's ranking of the GPU's norms."""
    banner(f"c2 weight-aware {name}")
    Wt, x, seg = make(name, seed=7)
    n_in, n_out = Wt.shape
    k_top, k_mid = pct_count(15, n_in), pct_count(35, n_in)
    rng = np.random.default_rng(n_in)
    # integer weights with per-channel spread, so the norm reorders channels
    Wi = np.round(rng.standard_normal((n_in, n_out)) * rng.uniform(0.3, 3.0, (n_in, 1)))
    Wi = synth.f32_to_bf16_bits(np.clip(Wi, -16, 16).astype(np.float32))
    y = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    proj = TieredProjection(dev(Wi), seg, k_top, k_mid, weight_aware=True)
    proj(dev(x), y)
    torch.cuda.synchronize()
    nrm = oracle.row_norms(Wi).astype(np.float32)
    assert np.array_equal(host(proj.norms).view(np.uint32), nrm.view(np.uint32))
    cnt = host(proj.cnt)
    top, mid = host(proj.idx_top)[:cnt[0]], host(proj.idx_mid)[:cnt[1]]
    o_top, o_mid = oracle.weighted_tier_sets(x, nrm, k_top, k_mid)
    assert np.array_equal(top, o_top) and np.array_equal(mid, o_mid)
    assert not np.array_equal(o_top, oracle.tier_sets(x, k_top, k_mid)[0])
    enc = oracle.encode_4bit(Wi, seg)
    assert_close(host(y), oracle.tiered_gemv(Wi, *enc, seg, x, o_top, o_mid), what="integer W")

    # the workload's weights: the norms are fp32 sums on the GPU and fp64 in
    # the oracle, so they are compared within rounding; the tiers are then
    # checked bit-exact with the oracle's ranking fed the GPU's own norms
    # (stage by stage: the select stage sees the bytes the GPU ranked)
    proj = TieredProjection(dev(Wt), seg, k_top, k_mid, weight_aware=True)
    proj(dev(x), y)
    torch.cuda.synchronize()
    ref_n = oracle.row_norms(Wt)
    gpu_n = host(proj.norms)
    np.testing.assert_allclose(gpu_n, ref_n, rtol=1e-5, atol=0)
    cnt = host(proj.cnt)
    top, mid = host(proj.idx_top)[:cnt[0]], host(proj.idx_mid)[:cnt[1]]
    assert top.size == k_top and mid.size == k_mid
    o_top, o_mid = oracle.weighted_tier_sets(x, gpu_n.astype(np.float32), k_top, k_mid)
    assert np.array_equal(top, o_top), (name, np.setxor1d(top, o_top))
    assert np.array_equal(mid, o_mid), (name, np.setxor1d(mid, o_mid))
    enc = oracle.encode_4bit(Wt, seg)
    assert_close(host(y), oracle.tiered_gemv(Wt, *enc, seg, x, top, mid), what="weight-aware")
