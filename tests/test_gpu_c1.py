"""SelectInfer stack (Llama3.2-3B FFN shape, 28 layers at full size):
calibration -> Eq (1) base sets, prefill -> per-token top-alpha, frequency
top-beta, union, then decode over the union, against the oracle stage by
stage (each oracle stage fed the GPU's inputs to that stage)."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import RMS_EPS, SelectInferStack, pct_count, to_device_bf16
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]


def run_stack(L, N, d, n_calib, n_prompt, n_decode, check_layers, check_tokens, seed=0):
    banner(f"c1 L={L} N={N} d={d} calib={n_calib} prompt={n_prompt} decode={n_decode}")
    layers = synth.ffn_stack(seed, synth.W_C1, L, N, d)
    dev_layers = [tuple(to_device_bf16(m) for m in lay) for lay in layers]
    base_k, alpha_k, beta_k = pct_count(20, N), pct_count(30, N), pct_count(20, N)
    stack = SelectInferStack(dev_layers, base_k, alpha_k, beta_k,
                             max_tokens=max(n_calib, n_prompt))
    Xc = synth.tokens(seed, synth.W_C1, 1, n_calib, d)
    Xp = synth.tokens(seed, synth.W_C1, 2, n_prompt, d)
    Xd = synth.tokens(seed, synth.W_C1, 3, n_decode, d)

    seen = {}

    def rec_calib(l, H, A):
        if l in check_layers:
            seen[("c", l)] = (host(H).copy(), host(A).copy())

    stack.calibrate(dev(Xc), record=rec_calib)
    torch.cuda.synchronize()
    scores = host(stack.scores)
    base_mask = host(stack.base_mask)
    for l in check_layers:
        Wg, Wu, WdT = layers[l]
        H, A = seen[("c", l)]
        for t in (0, n_calib // 2, n_calib - 1):
            x = oracle.rms_normalize(H[t], RMS_EPS)
            assert_close(A[t], oracle.swiglu_acts(Wg, Wu, x), what=f"calib A l={l} t={t}")
        s_ref, base_ref = oracle.base_set(A, base_k)
        assert np.array_equal(scores[l].view(np.uint32), s_ref.view(np.uint32)), l
        assert np.array_equal(np.flatnonzero(base_mask[l]), base_ref), l

    def rec_prompt(l, H, A):
        if l in check_layers:
            seen[("p", l)] = (host(H).copy(), host(A).copy())

    stack.prefill(dev(Xp), record=rec_prompt)
    torch.cuda.synchronize()
    freq = host_u32(stack.freq)
    U_cnt = host(stack.U_cnt)
    U_idx = host(stack.U_idx)
    for l in check_layers:
        Wg, Wu, WdT = layers[l]
        H, A = seen[("p", l)]
        x = oracle.rms_normalize(H[n_prompt - 1], RMS_EPS)
        assert_close(A[n_prompt - 1], oracle.swiglu_acts(Wg, Wu, x), what=f"prompt A l={l}")
        counts, dyn = oracle.dynamic_set(A, alpha_k, beta_k)
        assert np.array_equal(freq[l], counts.astype(np.uint32)), l
        U_ref = oracle.union(np.flatnonzero(base_mask[l]), dyn)
        assert U_cnt[l] == U_ref.size and np.array_equal(U_idx[l, :U_cnt[l]], U_ref), l
    print(f"  |U| per layer: min {U_cnt.min()} mean {U_cnt.mean():.1f} max {U_cnt.max()}")
    for l in check_layers:                        # per-prompt compaction, bit-exact
        Wg, Wu, WdT = layers[l]
        U = U_idx[l, :U_cnt[l]]
        gu, dT, _, k = stack.comp[l]
        gu_h = host(gu).view(np.uint16)
        dT_h = host(dT).view(np.uint16)
        assert k == U.size
        assert np.array_equal(gu_h[:, :d], Wg[U]) and np.array_equal(gu_h[:, d:], Wu[U])
        assert np.array_equal(dT_h[:, :k], WdT[U].T) and not dT_h[:, k:].any()

    for t in range(n_decode):
        h = dev(Xd[t])
        for l in range(L):
            check = t in check_tokens and l in check_layers
            h_in = host(h).copy() if check else None
            gathered = t == n_decode - 1          # last token: the uncompacted path
            if gathered:
                stack.decode_layer_gathered(l, h)
            else:
                stack.decode_layer(l, h)
            if check:
                torch.cuda.synchronize()
                Wg, Wu, WdT = layers[l]
                U = U_idx[l, :U_cnt[l]]
                a = host(stack.a[l])[U] if gathered else host(stack.comp[l][2])[:U.size]
                x = oracle.rms_normalize(h_in, RMS_EPS)
                assert_close(a, oracle.swiglu_acts(Wg, Wu, x, U), what=f"decode a t={t} l={l}")
                y_ref = oracle.down_gather(WdT, U, a)
                assert_close(host(h) - h_in, y_ref, what=f"decode y t={t} l={l}")
    torch.cuda.synchronize()
    return stack


def test_small_stack():
    run_stack(L=3, N=512, d=256, n_calib=64, n_prompt=32, n_decode=4,
              check_layers={0, 1, 2}, check_tokens={0, 3})


def test_full_size_stack():
    run_stack(L=28, N=8192, d=3072, n_calib=512, n_prompt=256, n_decode=128,
              check_layers={0, 13, 27}, check_tokens={0, 127})


def test_decode_graph_replays_match_eager():
    """The decode step captured as a HIP graph gives, on every replay, the
    bits the eager calls give (all reductions run in a fixed order)."""
    banner("c1 graph replay")
    L, N, d = 4, 1024, 512
    layers = synth.ffn_stack(5, synth.W_C1, L, N, d)
    dev_layers = [tuple(to_device_bf16(m) for m in lay) for lay in layers]
    stack = SelectInferStack(dev_layers, pct_count(20, N), pct_count(30, N), pct_count(20, N),
                             max_tokens=64)
    stack.calibrate(dev(synth.tokens(5, synth.W_C1, 1, 64, d)))
    stack.prefill(dev(synth.tokens(5, synth.W_C1, 2, 32, d)))
    X = dev(synth.tokens(5, synth.W_C1, 3, 6, d))
    eager = []
    for t in range(6):
        h = X[t].clone()
        stack.decode(h)
        eager.append(host(h))
    h = torch.zeros(d, dtype=torch.float32, device="cuda")
    xcur = torch.zeros(d, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.copy_(xcur)
        stack.decode(h)
    for rep in range(3):
        for t in range(6):
            xcur.copy_(X[t])
            g.replay()
            got = host(h)          # synchronizes between replays
            assert np.array_equal(got.view(np.uint32), eager[t].view(np.uint32)), (rep, t)
