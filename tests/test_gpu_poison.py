"""Skipped rows are never read: every weight row (and every per-row input:
activations, gates, biases) outside the selection is set to NaN, and the
gathered kernels must write bitwise what they write on clean data.  A NaN
that reached any sum would make the output NaN, so bitwise equality shows
the kernels read the selected rows only (SelectInfer §5 computes only the
selected neurons; the PowerInfer-2 guide's engine touches only the selected
clusters).  Covered: the batch-1 row ops over index lists on both kernel
shapes (SwiGLU, the gated up product and the fused ReGLU over 32-row
clusters, plain dots) and over several row lists, the batched MFMA row ops
over an index list, and the batched union contraction with rows outside the
union and each token's masked-out activations poisoned."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from gpu_common import assert_close, banner, dev, gpu, host, needs_gpu

pytestmark = [gpu, needs_gpu]

NAN_BF16 = np.uint16(0x7FC0)
SENTINEL = -7.25


def poison_rows(W, keep_rows):
    P = np.full_like(W, NAN_BF16)
    P[keep_rows] = W[keep_rows]
    return P


def poison_vec(v, keep, axis=-1):
    P = np.full_like(v, np.nan)
    if v.ndim == 1:
        P[keep] = v[keep]
    else:
        P[:, keep] = v[:, keep]
    return P


def bits(t):
    return host(t).view(np.uint32)


def rowop(op, W0, W1, x, n_out, idx, k_max, group=1, aux=None, batch=1, **kw):
    shape = (n_out,) if batch == 1 else (batch, n_out)
    out = torch.full(shape, SENTINEL, dtype=torch.float32, device="cuda")
    key = torch.full(shape, 12345, dtype=torch.int32, device="cuda")
    cnt = torch.tensor([len(idx)], dtype=torch.int32, device="cuda")
    B.sparse_ffn_gemv(op, None if W0 is None else dev(W0), None if W1 is None else dev(W1),
                      dev(x), out, idx=dev(idx), count=cnt, k_max=k_max, group=group,
                      aux=None if aux is None else dev(aux), key_out=key, **kw)
    torch.cuda.synchronize()
    return out, key


@pytest.mark.parametrize("d", [3072, 6144])
def test_batch1_rowops_never_read_skipped_rows(d):
    """d = 3072 takes the wave-per-row kernel, d = 6144 the workgroup-per-row kernel."""
    banner(f"poison batch-1 row ops d={d}")
    N = 2912   # 91 clusters of 32
    Wg = synth.weight_bf16(21, synth.W_C0, 9, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(21, synth.W_C0, 9, 0, synth.T_UP, N, d)
    x = synth.tokens(21, synth.W_C0, 9, 1, d)[0]
    rng = np.random.default_rng(d)

    # SwiGLU and plain dots over an index list
    sel = np.sort(rng.choice(N, size=1001, replace=False)).astype(np.int32)
    for op, W0, W1 in [(B.OP_GLU_SILU, Wg, Wu), (B.OP_DOT, Wg, None)]:
        clean, ck = rowop(op, W0, W1, x, N, sel, N)
        bad, bk = rowop(op, poison_rows(W0, sel), None if W1 is None else poison_rows(W1, sel),
                        x, N, sel, N)
        assert np.array_equal(bits(clean), bits(bad)), f"op {op}: a skipped row was read"
        assert np.array_equal(bits(ck), bits(bk))
        assert np.all(np.isfinite(host(bad)[sel]))
        assert np.all(host(bad)[np.setdiff1d(np.arange(N), sel)] == SENTINEL)
    ref = oracle.swiglu_acts(Wg, Wu, x, sel)
    assert_close(host(rowop(B.OP_GLU_SILU, Wg, Wu, x, N, sel, N)[0])[sel], ref, what="GLU")

    # the gated up product and the fused ReGLU over 32-row clusters
    clusters = np.sort(rng.choice(N // 32, size=23, replace=False)).astype(np.int32)
    rows = oracle.expand_clusters(clusters, 32)
    gate = rng.standard_normal(N).astype(np.float32)
    q = 1.2815515655446004 * synth.WEIGHT_STD
    cases = [
        (B.OP_GATED, None, Wu, dict(aux=gate)),
        (B.OP_GLU_RELU, Wg, Wu, dict(tau_scale=q, rms_eps=1e-5)),
    ]
    for op, W0, W1, kw in cases:
        aux = kw.pop("aux", None)
        clean, ck = rowop(op, W0, W1, x, N, clusters, N // 32, group=32, aux=aux, **kw)
        bad, bk = rowop(op, None if W0 is None else poison_rows(W0, rows), poison_rows(W1, rows),
                        x, N, clusters, N // 32, group=32,
                        aux=None if aux is None else poison_vec(aux, rows), **kw)
        assert np.array_equal(bits(clean), bits(bad)), f"op {op}: a skipped row was read"
        assert np.array_equal(bits(ck), bits(bk))
        assert np.all(np.isfinite(host(bad)[rows]))


def test_rowop_lists_never_read_skipped_rows():
    """Two row lists (two experts' clusters) in one launch: fused ReGLU and
    the gated up product, each expert's rows outside its clusters poisoned."""
    banner("poison row lists")
    N, d = 2048, 1024
    W = [synth.weight_bf16(22, synth.W_C3, 0, e, t, N, d) for e in range(2)
         for t in (synth.T_GATE, synth.T_UP)]
    x = synth.tokens(22, synth.W_C3, 0, 1, d)[0]
    rng = np.random.default_rng(5)
    cl = [np.sort(rng.choice(N // 32, size=k, replace=False)).astype(np.int32) for k in (9, 17)]
    rows = [oracle.expand_clusters(c, 32) for c in cl]
    gates = [rng.standard_normal(N).astype(np.float32) for _ in range(2)]
    q = 1.2815515655446004 * synth.WEIGHT_STD

    def run(op, Wg, Wu, aux):
        outs = [torch.full((N,), SENTINEL, dtype=torch.float32, device="cuda") for _ in range(2)]
        cnts = [torch.tensor([len(c)], dtype=torch.int32, device="cuda") for c in cl]
        B.sparse_ffn_rowop_lists(op, None if Wg is None else [dev(w) for w in Wg],
                                 [dev(w) for w in Wu], dev(x), outs,
                                 idxs=[dev(c) for c in cl], counts=cnts, k_maxs=[N // 32] * 2,
                                 group=32, tau_scale=q, rms_eps=1e-5,
                                 auxs=None if aux is None else [dev(a) for a in aux])
        torch.cuda.synchronize()
        return [bits(o) for o in outs]

    Wg, Wu = [W[0], W[2]], [W[1], W[3]]
    Pg = [poison_rows(Wg[e], rows[e]) for e in range(2)]
    Pu = [poison_rows(Wu[e], rows[e]) for e in range(2)]
    Pa = [poison_vec(gates[e], rows[e]) for e in range(2)]
    for e, (c, b) in enumerate(zip(run(B.OP_GLU_RELU, Wg, Wu, None),
                                   run(B.OP_GLU_RELU, Pg, Pu, None))):
        assert np.array_equal(c, b), f"ReGLU list {e}: a skipped row was read"
    for e, (c, b) in enumerate(zip(run(B.OP_GATED, None, Wu, gates),
                                   run(B.OP_GATED, None, Pu, Pa))):
        assert np.array_equal(c, b), f"gated list {e}: a skipped row was read"


@pytest.mark.parametrize("batch", [4, 16, 19])
def test_mfma_rowops_never_read_skipped_rows(batch):
    """Batched row ops over an index list that ends mid-tile (the last
    workgroup's dead items must re-read a selected row, not row 0)."""
    banner(f"poison MFMA row ops batch={batch}")
    N, d = 1500, 640
    Wg = synth.weight_bf16(23, synth.W_C4, 0, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(23, synth.W_C4, 0, 0, synth.T_UP, N, d)
    X = synth.tokens(23, synth.W_C4, 1, batch, d)
    rng = np.random.default_rng(batch)
    sel = np.sort(rng.choice(np.arange(1, N), size=531, replace=False)).astype(np.int32)
    assert 0 not in sel
    aux = rng.standard_normal((batch, N)).astype(np.float32)
    q = 1.2815515655446004 * synth.WEIGHT_STD
    cases = [
        (B.OP_GLU_SILU, Wg, Wu, None, {}),
        (B.OP_GATED, None, Wu, aux, {}),
        (B.OP_DOT_RELU, Wg, None, None, dict(tau_scale=q, rms_eps=1e-5)),
        (B.OP_DOT, Wg, None, None, {}),
    ]
    for op, W0, W1, ax, kw in cases:
        clean, ck = rowop(op, W0, W1, X, N, sel, N, aux=ax, batch=batch, **kw)
        bad, bk = rowop(op, None if W0 is None else poison_rows(W0, sel),
                        None if W1 is None else poison_rows(W1, sel), X, N, sel, N,
                        aux=None if ax is None else poison_vec(ax, sel), batch=batch, **kw)
        assert np.array_equal(bits(clean), bits(bad)), f"op {op}: a skipped row was read"
        assert np.array_equal(bits(ck), bits(bk))
        assert np.all(np.isfinite(host(bad)[:, sel]))
    got = host(rowop(B.OP_GLU_SILU, Wg, Wu, X, N, sel, N, batch=batch)[0])
    for b in (0, batch - 1):
        assert_close(got[b, sel], oracle.swiglu_acts(Wg, Wu, X[b], sel), what=f"GLU b={b}")


@pytest.mark.parametrize("batch", [4, 16, 19])
def test_union_contraction_never_reads_outside_union(batch):
    """The union contraction reads W_down^T rows of U only, and a token's
    activations outside its own selection only to zero them: rows outside U
    and every (token, neuron) activation outside S_b are NaN."""
    banner(f"poison union contraction batch={batch}")
    N, d = 4096, 1024
    WdT = synth.weight_bf16(24, synth.W_C4, 0, 0, synth.T_DOWN, N, d)
    rng = np.random.default_rng(100 + batch)
    U = np.sort(rng.choice(N, size=2111, replace=False)).astype(np.int32)
    M = np.zeros((batch, N), np.uint8)
    for b in range(batch):
        M[b, rng.choice(U, size=int(0.6 * U.size), replace=False)] = 1
    A = rng.standard_normal((batch, N)).astype(np.float32)
    cnt = torch.tensor([U.size], dtype=torch.int32, device="cuda")
    ws = B.new_workspace(batch, N, d)

    def run(W, Aa):
        Y = torch.full((batch, d), SENTINEL, dtype=torch.float32, device="cuda")
        B.sparse_ffn_gemv(B.OP_AXPY, dev(W), None, dev(Aa), Y, idx=dev(U), count=cnt, k_max=N,
                          row_mask=dev(M), workspace=ws)
        torch.cuda.synchronize()
        return Y

    clean = run(WdT, A)
    Ap = np.where(M != 0, A, np.float32(np.nan)).astype(np.float32)
    bad = run(poison_rows(WdT, U), Ap)
    assert np.array_equal(bits(clean), bits(bad)), "a row outside U or a masked activation was used"
    Y = host(bad)
    assert np.all(np.isfinite(Y))
    for b in range(batch):
        s = np.flatnonzero(M[b]).astype(np.int32)
        assert_close(Y[b], oracle.down_gather(WdT, s, A[b, s]), what=f"union output b={b}")
