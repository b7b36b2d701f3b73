"""Batch-1 row operations against the oracle on both kernel shapes: rows up
to 5120 wide take the wave-per-row kernel, wider rows the workgroup-per-row
kernel.  Widths cover ragged chunk counts, the wave kernel's limit and the
wider path; 2912 rows give several rows per wave.  Cases: SwiGLU with keys
(dense, with the fused RMSNorm, and over a gathered index list that leaves
other rows untouched), plain dots added to an output, the thresholded ReLU
gate and the gated product over 32-row clusters; tall single-matrix cases
give up to seven rows per wave."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]

WIDTHS = [520, 4104, 5120, 6144, 8192]
N = 2912            # 91 clusters of 32
EPS = 1e-5


def make(d, seed):
    W0 = synth.weight_bf16(seed, synth.W_C0, 9, 0, synth.T_GATE, N, d)
    W1 = synth.weight_bf16(seed, synth.W_C0, 9, 0, synth.T_UP, N, d)
    x = synth.tokens(seed, synth.W_C0, 9, 1, d)[0]
    return W0, W1, x


@pytest.mark.parametrize("d", WIDTHS)
def test_glu_dense_norm_and_gathered(d):
    banner(f"rowops glu d={d}")
    W0, W1, x = make(d, seed=11)
    a = torch.zeros(N, dtype=torch.float32, device="cuda")
    key = torch.zeros(N, dtype=torch.int32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(W0), dev(W1), dev(x), a, key_out=key)
    torch.cuda.synchronize()
    got = host(a)
    assert_close(got, oracle.swiglu_acts(W0, W1, x), what=f"dense GLU d={d}")
    assert np.array_equal(host_u32(key), oracle.key_abs(got)), "keys are not |a| bits"

    B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(W0), dev(W1), dev(x), a, rms_eps=EPS)
    torch.cuda.synchronize()
    xn = oracle.rms_normalize(x, EPS)
    assert_close(host(a), oracle.swiglu_acts(W0, W1, xn), what=f"GLU with RMSNorm d={d}")

    sel = np.sort(np.random.default_rng(d).choice(N, size=1001, replace=False)).astype(np.int32)
    cnt = torch.tensor([sel.size], dtype=torch.int32, device="cuda")
    g = torch.full((N,), 4321.0, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(W0), dev(W1), dev(x), g, idx=dev(sel), count=cnt,
                      k_max=sel.size)
    torch.cuda.synchronize()
    gg = host(g)
    assert np.all(gg[np.setdiff1d(np.arange(N), sel)] == 4321.0), "an unselected row was written"
    assert_close(gg[sel], oracle.swiglu_acts(W0, W1, x, sel), what=f"gathered GLU d={d}")


@pytest.mark.parametrize("d", WIDTHS)
def test_dot_relu_and_gated(d):
    banner(f"rowops dot/relu/gated d={d}")
    W0, W1, x = make(d, seed=12)
    rng = np.random.default_rng(d + 1)

    y0 = rng.standard_normal(N).astype(np.float32)
    y = dev(y0)
    B.sparse_ffn_gemv(B.OP_DOT, dev(W0), None, dev(x), y, accumulate=True)
    torch.cuda.synchronize()
    assert_close(host(y), y0 + oracle.row_dots(W0, x), what=f"dot + accumulate d={d}")

    q = 1.2815515655446004 * synth.WEIGHT_STD
    r = torch.zeros(N, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_DOT_RELU, dev(W0), None, dev(x), r, tau_scale=q, rms_eps=EPS)
    torch.cuda.synchronize()
    xn = oracle.rms_normalize(x, EPS)
    tau = oracle.relu_threshold(xn, 1.2815515655446004, synth.WEIGHT_STD)
    r_ref = oracle.relu_gate(W0, xn, tau)
    assert_close(host(r), r_ref, what=f"ReLU gate d={d}")

    clusters = np.sort(rng.choice(N // 32, size=37, replace=False)).astype(np.int32)
    rows = oracle.expand_clusters(clusters, 32)
    aux = rng.standard_normal(N).astype(np.float32)
    out = torch.full((N,), -9.0, dtype=torch.float32, device="cuda")
    cnt = torch.tensor([clusters.size], dtype=torch.int32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GATED, None, dev(W1), dev(x), out, idx=dev(clusters), count=cnt,
                      k_max=N // 32, group=32, aux=dev(aux), rms_eps=EPS)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(got[np.setdiff1d(np.arange(N), rows)] == -9.0), "a row outside the clusters was written"
    ref = aux[rows].astype(np.float64) * oracle.row_dots(W1, xn, rows)
    assert_close(got[rows], ref, what=f"gated product d={d}")


@pytest.mark.parametrize("n_rows", [40000, 57000])
def test_single_matrix_many_rows_per_wave(n_rows):
    """Single-matrix row ops keep two rows in flight per wave.  40000 and
    57000 rows give 4-5 and 6-7 rows per wave on the plain path (2048
    workgroups), a quarter of them gathered 4-5 and 6-7 on the gathered path
    (512 workgroups), so the two-buffer loop ends on either buffer and waves
    one row short of the others.  Dots, the ReLU gate and two row lists (bitwise
    what separate calls write) against the oracle."""
    banner(f"rowops single-matrix rows={n_rows}")
    d = 256
    W0 = synth.weight_bf16(13, synth.W_C0, 9, 0, synth.T_GATE, n_rows, d)
    x = synth.tokens(13, synth.W_C0, 9, 1, d)[0]
    rng = np.random.default_rng(n_rows)
    y0 = rng.standard_normal(n_rows).astype(np.float32)
    y = dev(y0)
    B.sparse_ffn_gemv(B.OP_DOT, dev(W0), None, dev(x), y, accumulate=True)
    torch.cuda.synchronize()
    assert_close(host(y), y0 + oracle.row_dots(W0, x), what=f"dot, {n_rows} rows")

    q = 1.2815515655446004 * synth.WEIGHT_STD
    r = torch.zeros(n_rows, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_DOT_RELU, dev(W0), None, dev(x), r, tau_scale=q, rms_eps=EPS)
    torch.cuda.synchronize()
    xn = oracle.rms_normalize(x, EPS)
    tau = oracle.relu_threshold(xn, 1.2815515655446004, synth.WEIGHT_STD)
    assert_close(host(r), oracle.relu_gate(W0, xn, tau), what=f"ReLU gate, {n_rows} rows")

    k = n_rows // 4
    sel = np.sort(rng.choice(n_rows, size=k, replace=False)).astype(np.int32)
    cnt = torch.tensor([k], dtype=torch.int32, device="cuda")
    g = torch.full((n_rows,), 4321.0, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_DOT, dev(W0), None, dev(x), g, idx=dev(sel), count=cnt, k_max=k)
    torch.cuda.synchronize()
    gg = host(g)
    assert np.all(gg[np.setdiff1d(np.arange(n_rows), sel)] == 4321.0), "an unselected row was written"
    assert_close(gg[sel], oracle.row_dots(W0, x, sel), what=f"gathered dot, {k} of {n_rows} rows")

    h = n_rows // 2
    Wd = dev(W0)
    halves = [Wd[:h], Wd[h:]]
    outs = [torch.zeros(h, dtype=torch.float32, device="cuda") for _ in range(2)]
    refs = [torch.zeros(h, dtype=torch.float32, device="cuda") for _ in range(2)]
    for l in range(2):
        B.sparse_ffn_gemv(B.OP_DOT, halves[l], None, dev(x), refs[l])
    B.sparse_ffn_rowop_lists(B.OP_DOT, halves, None, dev(x), outs)
    torch.cuda.synchronize()
    for l in range(2):
        assert np.array_equal(host_u32(outs[l]), host_u32(refs[l])), ("lists", l)
    assert_close(np.concatenate([host(o) for o in outs]), oracle.row_dots(W0, x),
                 what=f"two row lists, {n_rows} rows")


@pytest.mark.parametrize("op", ["glu", "dot_relu", "gated", "dot", "glu_relu", "predict"])
def test_rowop_lists_match_separate_calls(op):
    """One launch over several row lists writes, for each list, bitwise what
    a separate sparse_ffn_gemv call writes; rows outside a list keep their
    values; an empty list is allowed."""
    banner(f"rowop lists {op}")
    rng = np.random.default_rng(["glu", "dot_relu", "gated", "dot", "glu_relu", "predict"].index(op))
    N, d, S = 2048, 4096, 32
    code = {"glu": B.OP_GLU_SILU, "dot_relu": B.OP_DOT_RELU, "gated": B.OP_GATED, "dot": B.OP_DOT,
            "glu_relu": B.OP_GLU_RELU, "predict": B.OP_PREDICT}[op]
    tau = {"dot_relu": 0.0256, "glu_relu": 0.0256, "predict": 0.45}.get(op, 0.0)
    eps = 0.0 if op == "dot" else 1e-5
    n_l = 3
    W0 = [dev(synth.weight_bf16(8, synth.W_C3, 0, e, synth.T_GATE, N, d)) for e in range(n_l)]
    W1 = [dev(synth.weight_bf16(8, synth.W_C3, 0, e, synth.T_UP, N, d)) for e in range(n_l)]
    aux = [dev(rng.standard_normal(N).astype(np.float32)) for _ in range(n_l)]
    x = dev(synth.tokens(8, synth.W_C3, 3, 1, d)[0])
    use0, use1 = op != "gated", op in ("glu", "gated", "glu_relu")
    for clustered in (False, True):
        if clustered:
            counts = [17, 0, 40]
            sel = [np.sort(rng.choice(N // S, size=max(c, 1), replace=False)).astype(np.int32)
                   for c in counts]
            idx = [dev(s) for s in sel]
            cnt = [dev(np.array([c], np.int32)) for c in counts]
            kw = dict(k_max=N // S, group=S)
        outs = [torch.full((N,), 3.0, dtype=torch.float32, device="cuda") for _ in range(n_l)]
        keys = [torch.zeros(N, dtype=torch.int32, device="cuda") for _ in range(n_l)]
        ref = [o.clone() for o in outs]
        rkeys = [k.clone() for k in keys]
        for l in range(n_l):
            B.sparse_ffn_gemv(code, W0[l] if use0 else None, W1[l] if use1 else None, x, ref[l],
                              key_out=rkeys[l], tau_scale=tau, rms_eps=eps,
                              aux=aux[l] if op in ("gated", "predict") else None,
                              **(dict(idx=idx[l], count=cnt[l], **kw) if clustered else {}))
        B.sparse_ffn_rowop_lists(code, W0 if use0 else None, W1 if use1 else None, x, outs,
                                 key_outs=keys, tau_scale=tau, rms_eps=eps,
                                 auxs=aux if op in ("gated", "predict") else None,
                                 **(dict(idxs=idx, counts=cnt, k_maxs=[N // S] * n_l, group=S)
                                    if clustered else {}))
        torch.cuda.synchronize()
        for l in range(n_l):
            assert np.array_equal(host_u32(outs[l]), host_u32(ref[l])), (op, clustered, l)
            assert np.array_equal(host_u32(keys[l]), host_u32(rkeys[l])), (op, clustered, l)
        if clustered:
            assert np.all(host(outs[1]) == 3.0)


def test_dot_relu_cluster_keys():
    """DOT_RELU_CLUSTER: the outputs are DOT_RELU's bit for bit, and the
    cluster keys are the largest magnitude key of each cluster's nonzero
    rows, raised over what key_out held (as the oracle's cluster max key),
    both for one matrix and over several lists."""
    banner("dot_relu cluster keys")
    N, d, S = 2048, 4096, 32
    tau = 1.2815515655446004 * 0.02
    Ws = [synth.clustered_gate_bf16(10 + e, synth.W_C3, 0, e, N, d, S) for e in range(2)]
    x = dev(synth.tokens(10, synth.W_C3, 4, 1, d)[0])
    outs = [torch.zeros(N, dtype=torch.float32, device="cuda") for _ in range(2)]
    ref = [torch.zeros(N, dtype=torch.float32, device="cuda") for _ in range(2)]
    prev = np.zeros((2, N // S), np.uint32)
    prev[1, ::7] = 0x3F000000                         # pre-existing keys are raised, not replaced
    keys = [dev(prev[j].copy()) for j in range(2)]
    for j in range(2):
        B.sparse_ffn_gemv(B.OP_DOT_RELU, dev(Ws[j]), None, x, ref[j], tau_scale=tau, rms_eps=EPS)
    B.sparse_ffn_rowop_lists(B.OP_DOT_RELU_CLUSTER, [dev(w) for w in Ws], None, x, outs,
                             key_outs=keys, group=S, tau_scale=tau, rms_eps=EPS)
    single = torch.zeros(N // S, dtype=torch.int32, device="cuda")
    out1 = torch.zeros(N, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_DOT_RELU_CLUSTER, dev(Ws[0]), None, x, out1, key_out=single, group=S,
                      tau_scale=tau, rms_eps=EPS)
    torch.cuda.synchronize()
    for j in range(2):
        r = host(outs[j])
        assert np.array_equal(r.view(np.uint32), host_u32(ref[j]))
        exp = np.maximum(oracle.cluster_max_key(oracle.key_abs(r), S), prev[j])
        assert np.array_equal(host_u32(keys[j]), exp), j
        assert 0.05 < np.mean(exp != 0) < 0.6
    assert np.array_equal(host_u32(out1), host_u32(ref[0]))
    assert np.array_equal(host_u32(single), oracle.cluster_max_key(oracle.key_abs(host(ref[0])), S))


def test_dot_relu_cluster_keys_wide_rows():
    """DOT_RELU_CLUSTER on rows wider than the wave kernel's limit (the
    workgroup-per-row kernel): same outputs as DOT_RELU, oracle cluster keys."""
    banner("dot_relu cluster keys, wide rows")
    N, d, S = 1024, 6144, 32
    tau = 1.2815515655446004 * 0.02
    W = synth.clustered_gate_bf16(12, synth.W_C3, 0, 0, N, d, S)
    x = dev(synth.tokens(12, synth.W_C3, 5, 1, d)[0])
    out = torch.zeros(N, dtype=torch.float32, device="cuda")
    ref = torch.zeros(N, dtype=torch.float32, device="cuda")
    keys = torch.zeros(N // S, dtype=torch.int32, device="cuda")
    B.sparse_ffn_gemv(B.OP_DOT_RELU, dev(W), None, x, ref, tau_scale=tau, rms_eps=EPS)
    B.sparse_ffn_gemv(B.OP_DOT_RELU_CLUSTER, dev(W), None, x, out, key_out=keys, group=S,
                      tau_scale=tau, rms_eps=EPS)
    torch.cuda.synchronize()
    r = host(out)
    assert np.array_equal(r.view(np.uint32), host_u32(ref))
    assert np.array_equal(host_u32(keys), oracle.cluster_max_key(oracle.key_abs(r), S))
    assert np.any(host_u32(keys)) and not np.all(host_u32(keys))


def test_rowop_lists_eight_lists():
    """The maximum of eight lists, with ragged counts (one empty), against
    one call per list, bitwise."""
    banner("rowop lists x8")
    rng = np.random.default_rng(13)
    N, d, S = 1024, 2048, 32
    Wg = [dev(synth.weight_bf16(13, synth.W_C3, 1, e, synth.T_GATE, N, d)) for e in range(8)]
    Wu = [dev(synth.weight_bf16(13, synth.W_C3, 1, e, synth.T_UP, N, d)) for e in range(8)]
    x = dev(synth.tokens(13, synth.W_C3, 6, 1, d)[0])
    counts = [5, 0, 32, 17, 1, 9, 23, 2]
    idx = [dev(np.sort(rng.choice(N // S, size=32, replace=False)).astype(np.int32)) for _ in range(8)]
    cnt = [dev(np.array([c], np.int32)) for c in counts]
    outs = [torch.full((N,), -2.0, dtype=torch.float32, device="cuda") for _ in range(8)]
    refs = [o.clone() for o in outs]
    for l in range(8):
        B.sparse_ffn_gemv(B.OP_GLU_RELU, Wg[l], Wu[l], x, refs[l], idx=idx[l], count=cnt[l],
                          k_max=N // S, group=S, tau_scale=0.02, rms_eps=EPS)
    B.sparse_ffn_rowop_lists(B.OP_GLU_RELU, Wg, Wu, x, outs, idxs=idx, counts=cnt,
                             k_maxs=[N // S] * 8, group=S, tau_scale=0.02, rms_eps=EPS)
    torch.cuda.synchronize()
    for l in range(8):
        assert np.array_equal(host_u32(outs[l]), host_u32(refs[l])), l
    assert np.all(host(outs[1]) == -2.0)
