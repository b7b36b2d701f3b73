"""Packed weight layouts of the batched kernels (sparse_ffn_pack_weights and
the SFFN_PACKED op flag).  The packed copies are checked element by element
against the layouts' definitions written out in numpy; the batched row ops
and the union contraction on packed weights give bitwise the results of the
row-major weights (same rows, same arithmetic, same order), dense and over
index lists, through the K-sliced path, with per-token masks, and with rows
outside the processed set NaN-poisoned; the packed batched layer is checked
against the oracle at the full C4 shape."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import BatchedUnionLayer, pct_count
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]

NAN_BF16 = np.uint16(0x7FC0)


def weights(N, d, tensor, seed):
    return synth.weight_bf16(seed, synth.W_C4, 3, 0, tensor, N, d)


def row_tiles_ref(W):
    """[ceil(n/16)][d/128][16][128], rows past n zero."""
    n, d = W.shape
    T = (n + 15) // 16
    P = np.zeros((T * 16, d), dtype=W.dtype)
    P[:n] = W
    return P.reshape(T, 16, d // 128, 128).transpose(0, 2, 1, 3).reshape(-1)


def col_panels_ref(W):
    """[d/256][n][256]."""
    n, d = W.shape
    return W.reshape(n, d // 256, 256).transpose(1, 0, 2).reshape(-1)


def u16(t):
    return host(t).view(np.uint16)


@pytest.mark.parametrize("n,d", [(1000, 384), (16, 128), (17408, 5120), (1, 256)])
def test_pack_layouts(n, d):
    banner(f"pack n={n} d={d}")
    W = weights(n, d, synth.T_GATE, seed=n + d)
    Wd = dev(W)
    pt = B.pack_weights(Wd, B.LAYOUT_ROW_TILES)
    assert pt.data.numel() == B.packed_elems(n, d, B.LAYOUT_ROW_TILES)
    assert np.array_equal(u16(pt.data), row_tiles_ref(W))
    if d % 256 == 0:
        pc = B.pack_weights(Wd, B.LAYOUT_COL_PANELS)
        assert np.array_equal(u16(pc.data), col_panels_ref(W))
    # a strided source (ld_w > d)
    wide = torch.zeros(n, d + 64, dtype=torch.int16, device="cuda")
    wide[:, :d] = Wd
    pt2 = B.pack_weights(wide[:, :d], B.LAYOUT_ROW_TILES)
    assert np.array_equal(u16(pt2.data), row_tiles_ref(W))


def rowop_pair(op, W0, W1, X, N, *, idx=None, k_max=0, aux=None, eps=0.0, ws=None, key=True):
    """The op on row-major and on packed weights; returns both (out, key)."""
    res = []
    for packed in (False, True):
        w0 = None if W0 is None else (B.pack_weights(W0, B.LAYOUT_ROW_TILES) if packed else W0)
        w1 = None if W1 is None else (B.pack_weights(W1, B.LAYOUT_ROW_TILES) if packed else W1)
        out = torch.full((X.shape[0], N), 3.25, dtype=torch.float32, device="cuda")
        k = torch.zeros(X.shape[0], N, dtype=torch.int32, device="cuda") if key else None
        cnt = None if idx is None else torch.tensor([k_max], dtype=torch.int32, device="cuda")
        B.sparse_ffn_gemv(op, w0, w1, X, out, idx=idx, count=cnt, k_max=k_max, aux=aux,
                          rms_eps=eps, tau_scale=0.05 if op == B.OP_DOT_RELU else 0.0,
                          key_out=k, workspace=ws)
        torch.cuda.synchronize()
        res.append((host(out), None if k is None else host_u32(k)))
    return res


@pytest.mark.parametrize("batch", [4, 16, 19])
def test_row_ops_packed_bitwise(batch):
    """Every batched row op, dense through the K-sliced path (8240 rows =
    258 tile pairs, with a workspace) and over an index list, on packed
    weights: bitwise the row-major results; GLU also against the oracle."""
    banner(f"packed row ops batch={batch}")
    N, d = 8240, 1024
    Wg, Wu = weights(N, d, synth.T_GATE, 1), weights(N, d, synth.T_UP, 1)
    X = synth.tokens(batch, synth.W_C4, 11, batch, d)
    aux = np.random.default_rng(batch).standard_normal((batch, N)).astype(np.float32)
    Xd, G, U, AUX = dev(X), dev(Wg), dev(Wu), dev(aux)
    ws = B.new_workspace(batch, N, d)
    sel = np.sort(np.random.default_rng(7).choice(N, 3001, replace=False)).astype(np.int32)
    for op, W0, W1 in ((B.OP_GLU_SILU, G, U), (B.OP_DOT_RELU, G, None), (B.OP_GATED, None, U),
                       (B.OP_DOT, G, None)):
        for eps in (0.0, 1e-5):
            (o0, k0), (o1, k1) = rowop_pair(op, W0, W1, Xd, N, aux=AUX if op == B.OP_GATED else None,
                                            eps=eps, ws=ws)
            assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), (op, eps)
            assert np.array_equal(k0, k1), (op, eps)
        (o0, _), (o1, _) = rowop_pair(op, W0, W1, Xd, N, idx=dev(sel), k_max=sel.size,
                                      aux=AUX if op == B.OP_GATED else None, key=False)
        assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), (op, "gathered")
        skipped = np.setdiff1d(np.arange(N), sel)
        assert np.all(o1[:, skipped] == 3.25), "a row outside the index list was written"
    (o1, _), = rowop_pair(B.OP_GLU_SILU, G, U, Xd, N, ws=ws, key=False)[1:]
    for t in (0, batch - 1):
        assert_close(o1[t], oracle.swiglu_acts(Wg, Wu, X[t]), what=f"packed GLU token {t}")


@pytest.mark.parametrize("batch,N,d", [(4, 3000, 512), (16, 3000, 512), (16, 17408, 5120)])
def test_union_contraction_packed_bitwise(batch, N, d):
    """The batched AXPY over an index list with per-token masks on packed
    column panels: bitwise the row-major result, rows outside the list
    NaN-poisoned, and against the oracle over each token's own rows."""
    banner(f"packed union contraction batch={batch} N={N} d={d}")
    WdT = weights(N, d, synth.T_DOWN, seed=batch)
    rng = np.random.default_rng(N + batch)
    A = rng.standard_normal((batch, N)).astype(np.float32)
    M = (rng.random((batch, N)) < 0.4).astype(np.uint8)
    U = np.flatnonzero(M.any(axis=0)).astype(np.int32)
    pad = min(37, N - U.size)                    # index entries past the count (unused)
    k_max = U.size + pad
    idx = np.concatenate([U, np.zeros(pad, np.int32)])
    cnt = torch.tensor([U.size], dtype=torch.int32, device="cuda")
    ws = B.new_workspace(batch, N, d)

    def run(W, packed):
        w = B.pack_weights(dev(W), B.LAYOUT_COL_PANELS) if packed else dev(W)
        Y = torch.zeros(batch, d, dtype=torch.float32, device="cuda")
        B.sparse_ffn_gemv(B.OP_AXPY, w, None, dev(A), Y, idx=dev(idx), count=cnt, k_max=k_max,
                          row_mask=dev(M), workspace=ws)
        torch.cuda.synchronize()
        return host(Y)

    y0, y1 = run(WdT, False), run(WdT, True)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    P = np.full_like(WdT, NAN_BF16)
    P[U] = WdT[U]
    yp = run(P, True)
    assert np.all(np.isfinite(yp)) and np.array_equal(yp.view(np.uint32), y1.view(np.uint32))
    for b in (0, batch - 1):
        s = np.flatnonzero(M[b])
        assert_close(y1[b], oracle.down_gather(WdT, s, A[b][s]), what=f"packed AXPY token {b}")


@pytest.mark.parametrize("batch", [4, 16])
def test_packed_batched_layer_full_size(batch):
    """The batched union layer on packed weights at the 17408 x 5120 shape:
    the same bits as the row-major layer, and the oracle's activations, index
    sets and outputs for sampled tokens."""
    banner(f"packed batched layer batch={batch}")
    N, d = 17408, 5120
    Wg = synth.weight_bf16(0, synth.W_C4, 0, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(0, synth.W_C4, 0, 0, synth.T_UP, N, d)
    WdT = synth.weight_bf16(0, synth.W_C4, 0, 0, synth.T_DOWN, N, d)
    X = synth.tokens(0, synth.W_C4, batch, batch, d)
    keep = pct_count(40, N)
    G, U, D = dev(Wg), dev(Wu), dev(WdT)
    outs = []
    for packed in (False, True):
        layer = BatchedUnionLayer(G, U, D, keep, batch, packed=packed)
        Y = torch.zeros(batch, d, dtype=torch.float32, device="cuda")
        layer(dev(X), Y)
        torch.cuda.synchronize()
        outs.append((host(layer.A), host(layer.M), host(Y)))
    (A0, M0, Y0), (A1, M1, Y1) = outs
    assert np.array_equal(A0.view(np.uint32), A1.view(np.uint32))
    assert np.array_equal(M0, M1)
    assert np.array_equal(Y0.view(np.uint32), Y1.view(np.uint32))
    for b in (0, batch - 1):
        assert_close(A1[b], oracle.swiglu_acts(Wg, Wu, X[b]), what=f"activations b={b}")
        s = oracle.rank_range(oracle.key_abs(A1[b]), 0, keep)
        assert np.array_equal(np.flatnonzero(M1[b]), s), b
        assert_close(Y1[b], oracle.down_gather(WdT, s, A1[b][s]), what=f"output b={b}")
