"""Batched decode (Qwen-27B-like layer at full size, batch 1/4/8/16):
per-token top-k, union gathered once, MFMA contraction with per-token
masks, against the oracle stage by stage."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import BatchedUnionLayer, pct_count, threshold_members
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]


def make(N, d, batch, seed=0):
    Wg = synth.weight_bf16(seed, synth.W_C4, 0, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(seed, synth.W_C4, 0, 0, synth.T_UP, N, d)
    WdT = synth.weight_bf16(seed, synth.W_C4, 0, 0, synth.T_DOWN, N, d)
    X = synth.tokens(seed, synth.W_C4, batch, batch, d)
    return Wg, Wu, WdT, X


def run_and_check(N, d, batch, pct, seed=0, sample_tokens=None, union_list=False):
    Wg, Wu, WdT, X = make(N, d, batch, seed)
    keep = pct_count(pct, N)
    # at batch 1 union_list picks the listed path (index list + listed
    # product) over the keyed one (threshold + keyed product)
    layer = BatchedUnionLayer(dev(Wg), dev(Wu), dev(WdT), keep, batch, union_list=union_list,
                              keyed=not union_list)
    keyed = layer.keyed
    # the union as an index list exists on the listed batch-1 path and with
    # union_list; the keyed product reads a threshold, the masked product
    # forms the union from the token masks, neither lists it
    listed = (batch == 1 and not keyed) or union_list
    Y = torch.zeros(batch, d, dtype=torch.float32, device="cuda")
    layer(dev(X), Y)
    torch.cuda.synchronize()
    A = host(layer.A)
    K = host_u32(layer.K)
    M = host(layer.M)
    F = host_u32(layer.F)
    if keyed:
        U = threshold_members(K[0], host(layer.thr))
        cnt = U.size
    else:
        cnt = int(host(layer.cnt)[0]) if listed else int(M.any(axis=0).sum())
        U = host(layer.U)[:cnt] if listed else np.flatnonzero(M.any(axis=0))
    toks = range(batch) if sample_tokens is None else sample_tokens
    for b in toks:
        assert_close(A[b], oracle.swiglu_acts(Wg, Wu, X[b]), what=f"activations b={b}")
    S = []
    for b in range(batch):
        assert np.array_equal(K[b], oracle.key_abs(A[b]))
        s = oracle.rank_range(oracle.key_abs(A[b]), 0, keep)
        if not keyed:   # (the keyed path writes no masks)
            m = np.zeros(N, np.uint8)
            m[s] = 1
            assert np.array_equal(M[b], m), b
        S.append(s)
    U_ref = oracle.union(*S)
    assert np.array_equal(U, U_ref)
    # the frequency counts were consumed by the union select and reset
    assert not F.any()
    for b in toks:
        y_ref = oracle.down_gather(WdT, S[b], A[b][S[b]])
        assert_close(host(Y[b]), y_ref, what=f"output b={b}")
    print(f"  union {cnt} of {N} ({cnt / N:.3f})")
    # a second batch on other tokens: its union starts from the reset counts
    X2 = synth.tokens(seed, synth.W_C4, batch + 100, batch, d)
    layer(dev(X2), Y)
    torch.cuda.synchronize()
    A2 = host(layer.A)
    S2 = [oracle.rank_range(oracle.key_abs(A2[b]), 0, keep) for b in range(batch)]
    if keyed:
        assert np.array_equal(threshold_members(host_u32(layer.K)[0], host(layer.thr)),
                              oracle.union(*S2))
    elif listed:
        cnt2 = int(host(layer.cnt)[0])
        assert np.array_equal(host(layer.U)[:cnt2], oracle.union(*S2))
    else:
        M2 = host(layer.M)
        assert np.array_equal(np.flatnonzero(M2.any(axis=0)), oracle.union(*S2))
    for b in toks:
        assert_close(host(Y[b]), oracle.down_gather(WdT, S2[b], A2[b][S2[b]]),
                     what=f"second batch output b={b}")
    return layer, Y


@pytest.mark.parametrize("union_list", [False, True])
@pytest.mark.parametrize("batch", [1, 2, 4, 8, 16, 19])
def test_small_shapes(batch, union_list):
    banner(f"c4 small batch={batch} union_list={union_list}")
    run_and_check(1000, 256, batch, 40, seed=batch, union_list=union_list)


@pytest.mark.parametrize("union_list", [False, True])
@pytest.mark.parametrize("batch", [1, 4, 8, 16])
def test_full_size(batch, union_list):
    banner(f"c4 full batch={batch} union_list={union_list}")
    run_and_check(17408, 5120, batch, 40, sample_tokens=[0, batch - 1], union_list=union_list)


def test_mfma_dense_prefill_shape():
    """The dense batched path used by prefill / calibration (M = 256 tokens,
    no index list), against a plain fp64 product."""
    banner("c4 dense M=256")
    N, d, T = 1024, 512, 256
    Wg, Wu, WdT, _ = make(N, d, 1, seed=9)
    X = synth.tokens(9, synth.W_C4, 77, T, d)
    A = torch.zeros(T, N, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(Wg), dev(Wu), dev(X), A)
    H = dev(X).clone()
    ws = B.new_workspace(T, N, d)
    B.sparse_ffn_gemv(B.OP_AXPY, dev(WdT), None, A, H, accumulate=True, workspace=ws)
    torch.cuda.synchronize()
    A_ref, Y_ref = oracle.dense_ffn(Wg, Wu, WdT, X)
    for t in (0, 100, 255):
        assert_close(host(A[t]), oracle.swiglu_acts(Wg, Wu, X[t]), what=f"A[{t}]")
        y_ref = oracle.widen_bf16(WdT).T @ host(A[t]).astype(np.float64)
        assert_close(host(H[t]) - X[t], y_ref, what=f"H[{t}]")


@pytest.mark.parametrize("d", [96, 288, 416])
def test_mfma_rowop_ragged_k(d):
    """The batched row op walks K in 128-wide chunks and finishes the rest
    32 at a time: d below one chunk (96) and with a 32 / 32+128k tail,
    with and without the fused RMSNorm of each token's input, over a
    gathered index list that ends mid-tile."""
    banner(f"c4 ragged K d={d}")
    N, T = 200, 21
    Wg, Wu, _, _ = make(N, d, 1, seed=d)
    X = synth.tokens(d, synth.W_C4, 5, T, d)
    rows = np.sort(np.random.default_rng(d).choice(N, 77, replace=False)).astype(np.int32)
    idx = dev(rows)
    cnt = torch.tensor([len(rows)], dtype=torch.int32, device="cuda")
    for eps in (0.0, 1e-5):
        A = torch.full((T, N), 7.0, dtype=torch.float32, device="cuda")
        B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(Wg), dev(Wu), dev(X), A, idx=idx, count=cnt,
                          k_max=len(rows), rms_eps=eps)
        torch.cuda.synchronize()
        A_h = host(A)
        skipped = np.setdiff1d(np.arange(N), rows)
        assert np.all(A_h[:, skipped] == 7.0), "rows outside the index list were written"
        for t in range(T):
            x = oracle.rms_normalize(X[t], eps) if eps > 0 else X[t]
            assert_close(A_h[t, rows], oracle.swiglu_acts(Wg, Wu, x, rows),
                         what=f"d={d} eps={eps} token {t}")


@pytest.mark.parametrize("d,batch", [(416, 16), (1024, 19)])
def test_mfma_rowop_k_slices(d, batch):
    """With a workspace, a batched dense row op whose 32-row tile pairs do
    not split evenly over the CUs runs the last pairs as K slices plus a
    fix-up: 8240 rows = 258 pairs (the last with one live tile), d = 416
    (three 128-chunks and a 32-wide remainder, taken by the last slice) and
    1024; every op, with the fused RMSNorm where it applies, against the
    oracle; two sliced runs are bitwise equal."""
    banner(f"c4 K-sliced row ops d={d} batch={batch}")
    N = 8240
    Wg, Wu, _, _ = make(N, d, 1, seed=d + batch)
    X = synth.tokens(d, synth.W_C4, 7, batch, d)
    rng = np.random.default_rng(d)
    aux = rng.standard_normal((batch, N)).astype(np.float32)
    ws = B.new_workspace(batch, N, d)
    q = 1.2815515655446004 * synth.WEIGHT_STD
    cases = [(B.OP_GLU_SILU, dict(rms_eps=1e-5)), (B.OP_GLU_SILU, {}), (B.OP_DOT_RELU,
             dict(tau_scale=q, rms_eps=1e-5)), (B.OP_GATED, dict(rms_eps=1e-5)), (B.OP_DOT, {})]
    for op, kw in cases:
        outs = []
        for _ in range(2):
            A = torch.full((batch, N), 3.0, dtype=torch.float32, device="cuda")
            Kk = torch.zeros((batch, N), dtype=torch.int32, device="cuda")
            B.sparse_ffn_gemv(op, None if op == B.OP_GATED else dev(Wg),
                              dev(Wu) if op in (B.OP_GLU_SILU, B.OP_GATED) else None, dev(X), A,
                              aux=dev(aux) if op == B.OP_GATED else None, key_out=Kk,
                              workspace=ws, **kw)
            torch.cuda.synchronize()
            outs.append((host(A), host_u32(Kk)))
        assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32)), op
        A_h, K_h = outs[0]
        assert np.array_equal(K_h, oracle.key_abs(A_h)), op
        eps = kw.get("rms_eps", 0.0)
        for b in (0, batch // 2, batch - 1):
            x = oracle.rms_normalize(X[b], eps) if eps > 0 else X[b].astype(np.float64)
            if op == B.OP_GLU_SILU:
                ref = oracle.swiglu_acts(Wg, Wu, x)
            elif op == B.OP_DOT_RELU:
                ref = oracle.relu_gate(Wg, x, oracle.relu_threshold(x, 1.2815515655446004,
                                                                     synth.WEIGHT_STD))
            elif op == B.OP_GATED:
                ref = aux[b].astype(np.float64) * oracle.row_dots(Wu, x)
            else:
                ref = oracle.row_dots(Wg, x)
            assert_close(A_h[b], ref, what=f"op {op} eps {eps} token {b}")


@pytest.mark.parametrize("batch,packed", [(4, False), (16, True)])
def test_batched_layer_graph_replays_match_eager(batch, packed):
    """The batched layer (union formed inside the product; row-major or
    packed weights) captured as a HIP graph gives, on every replay, the bits
    the eager calls give, with other work and synchronisations between the
    replays."""
    banner(f"c4 graph replay batch={batch} packed={packed}")
    N, d = 3000, 512
    Wg, Wu, WdT, _ = make(N, d, 1, seed=31)
    layer = BatchedUnionLayer(dev(Wg), dev(Wu), dev(WdT), pct_count(40, N), batch, packed=packed)
    X = [dev(synth.tokens(31, synth.W_C4, 200 + t, batch, d)) for t in range(4)]
    eager = []
    for t in range(4):
        Y = torch.zeros(batch, d, dtype=torch.float32, device="cuda")
        layer(X[t], Y)
        eager.append(host(Y))
    xb = torch.zeros(batch, d, dtype=torch.float32, device="cuda")
    Y = torch.zeros(batch, d, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(xb, Y)
    for rep in range(3):
        for t in range(4):
            xb.copy_(X[t])
            g.replay()
            got = host(Y)          # synchronizes between replays
            assert np.array_equal(got.view(np.uint32), eager[t].view(np.uint32)), (rep, t)
            layer(X[(t + 1) % 4], torch.empty_like(Y))   # eager work between replays
