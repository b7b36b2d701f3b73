"""SelectInfer with selective loading, fill-to-phi and the Table 1 layer
range (Llama3.2-3B FFN shape, 28 layers at full size): profiling -> task
and model-specific Eq (1) scores, loading -> base and loaded sets and the
resident weights, prefill over the loaded neurons -> counts and the
computed set, then decode; against the oracle stage by stage (each oracle
stage fed the GPU's inputs to that stage)."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import (RMS_EPS, SelectInferLoadedStack, pct_count,
                                                    to_device_bf16)
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]


def run_loaded(L, N, d, n_task, n_mix, n_prompt, n_decode, first, last, check_layers,
               check_tokens, pcts=(30, 70, 30, 40), seed=0):
    delta_pct, gamma_pct, alpha_pct, phi_pct = pcts
    banner(f"c1-loading L={L} N={N} d={d} first={first} last={last} pcts={pcts}")
    layers = synth.ffn_stack(seed, synth.W_C1, L, N, d)
    dev_layers = [tuple(to_device_bf16(m) for m in lay) for lay in layers]
    dk, gk = pct_count(delta_pct, N), pct_count(gamma_pct, N)
    ak, pk = pct_count(alpha_pct, N), pct_count(phi_pct, N)
    stack = SelectInferLoadedStack(dev_layers, dk, gk, ak, pk, first=first, last=last,
                                   max_tokens=max(n_task, 3 * n_mix, n_prompt))
    modified = set(oracle.modified_layers(L, first, last))
    assert stack.modified == modified
    Xt = synth.tokens(seed, synth.W_C1, 11, n_task, d)
    Xm = synth.mixture_tokens(seed, synth.W_C1, 12, n_mix, d)
    Xp = synth.tokens(seed, synth.W_C1, 13, n_prompt, d)
    Xd = synth.tokens(seed, synth.W_C1, 14, n_decode, d)

    seen = {}

    def rec_profile(kind, l, H, A):
        if l in check_layers:
            seen[(kind, l)] = (host(H).copy(), host(A).copy())

    stack.profile(dev(Xt), dev(Xm), record=rec_profile)
    torch.cuda.synchronize()
    s_task, s_model = host(stack.s_task), host(stack.s_model)
    for kind, S in (("task", s_task), ("model", s_model)):
        for l in check_layers:
            Wg, Wu, _ = layers[l]
            H, A = seen[(kind, l)]
            t = H.shape[0] - 1
            assert_close(A[t], oracle.swiglu_acts(Wg, Wu, oracle.rms_normalize(H[t], RMS_EPS)),
                         what=f"{kind} A l={l}")
            assert np.array_equal(S[l].view(np.uint32), oracle.eq1_scores(A).view(np.uint32)), l

    stack.load()
    torch.cuda.synchronize()
    base_mask, load_idx, load_cnt = host(stack.base_mask), host(stack.load_idx), host(stack.load_cnt)
    static_mask = host(stack.static_mask)
    loaded_sets = {}
    for l in sorted(modified):
        base, loaded = oracle.selective_loading(s_task[l], s_model[l], dk, gk)
        assert np.array_equal(np.flatnonzero(base_mask[l]), base), l
        assert load_cnt[l] == loaded.size and np.array_equal(load_idx[l, :loaded.size], loaded), l
        static = oracle.loaded_positions(loaded, base)
        assert np.array_equal(np.flatnonzero(static_mask[l, :loaded.size]), static), l
        loaded_sets[l] = (loaded, static)
        if l in check_layers:                      # resident weights: the loaded rows, bit-exact
            Wg, Wu, WdT = layers[l]
            g_, u_, dn, _ = stack.resident[l]
            assert np.array_equal(host(g_).view(np.uint16), Wg[loaded])
            assert np.array_equal(host(u_).view(np.uint16), Wu[loaded])
            assert np.array_equal(host(dn).view(np.uint16), WdT[loaded])
    print(f"  loaded {gk} of {N} neurons in {len(modified)} of {L} layers")

    def rec_prompt(l, H, A):
        if l in check_layers:
            seen[("p", l)] = (host(H).copy(), host(A).copy())

    stack.prefill(dev(Xp), record=rec_prompt)
    torch.cuda.synchronize()
    freq = host_u32(stack.freq)
    U_pos, U_cnt = host(stack.U_pos), host(stack.U_cnt)
    computed = {}
    for l in range(L):
        if l in modified:
            loaded, static = loaded_sets[l]
            if l in check_layers:
                Wg, Wu, _ = layers[l]
                H, A = seen[("p", l)]
                x = oracle.rms_normalize(H[n_prompt - 1], RMS_EPS)
                assert_close(A[n_prompt - 1], oracle.swiglu_acts(Wg, Wu, x, loaded),
                             what=f"prompt A over loaded l={l}")
                counts, _ = oracle.dynamic_set(A, ak, 0)
                assert np.array_equal(freq[l, :loaded.size], counts.astype(np.uint32)), l
                U = oracle.fill_to_phi(static, counts, pk)
                assert U_cnt[l] == U.size and np.array_equal(U_pos[l, :U_cnt[l]], U), l
            computed[l] = loaded[U_pos[l, :U_cnt[l]]]
            assert computed[l].size == max(dk, min(pk, loaded.size)), l
        else:
            computed[l] = np.arange(N, dtype=np.int32)
            if l in check_layers:
                Wg, Wu, _ = layers[l]
                H, A = seen[("p", l)]
                x = oracle.rms_normalize(H[0], RMS_EPS)
                assert_close(A[0], oracle.swiglu_acts(Wg, Wu, x), what=f"prompt A dense l={l}")
    for l in check_layers:                          # per-prompt compaction, bit-exact
        Wg, Wu, WdT = layers[l]
        ids = computed[l]
        W0, W1, dT, _, k = stack.comp[l]
        assert k == ids.size
        assert np.array_equal(host(W0).view(np.uint16), Wg[ids])
        assert np.array_equal(host(W1).view(np.uint16), Wu[ids])
        dT_h = host(dT).view(np.uint16)
        assert np.array_equal(dT_h[:, :k], WdT[ids].T) and not dT_h[:, k:].any()

    for t in range(n_decode):
        h = dev(Xd[t])
        for l in range(L):
            check = t in check_tokens and l in check_layers
            h_in = host(h).copy() if check else None
            stack.decode_layer(l, h)
            if check:
                torch.cuda.synchronize()
                Wg, Wu, WdT = layers[l]
                ids = computed[l]
                a = host(stack.comp[l][3])[:ids.size]
                x = oracle.rms_normalize(h_in, RMS_EPS)
                assert_close(a, oracle.swiglu_acts(Wg, Wu, x, ids), what=f"decode a t={t} l={l}")
                assert_close(host(h) - h_in, oracle.down_gather(WdT, ids, a),
                             what=f"decode y t={t} l={l}")
    torch.cuda.synchronize()
    return stack


def test_small_loaded_stack():
    run_loaded(L=6, N=1024, d=512, n_task=64, n_mix=32, n_prompt=32, n_decode=4, first=1, last=-1,
               check_layers={0, 1, 3, 4, 5}, check_tokens={0, 3})


def test_degenerate_budgets():
    # only the base set loaded and computed; then phi at the base size (no dynamic neurons)
    run_loaded(L=3, N=520, d=256, n_task=32, n_mix=16, n_prompt=16, n_decode=2, first=0, last=0,
               check_layers={0, 1, 2}, check_tokens={1}, pcts=(30, 30, 30, 40))
    run_loaded(L=3, N=520, d=256, n_task=32, n_mix=16, n_prompt=16, n_decode=2, first=0, last=0,
               check_layers={0, 2}, check_tokens={1}, pcts=(25, 100, 10, 25))


def test_full_size_table1_stack():
    cfg = synth.SHAPES["c1_loading"]
    run_loaded(L=cfg["layers"], N=cfg["n"], d=cfg["d"], n_task=cfg["task_tokens"],
               n_mix=cfg["mixture_tokens_per_task"], n_prompt=cfg["prompt_tokens"],
               n_decode=cfg["decode_tokens"], first=cfg["first"], last=cfg["last"],
               check_layers={0, 5, 15, 25, 27}, check_tokens={0, 127},
               pcts=(cfg["base_pct"], cfg["loaded_pct"], cfg["alpha_pct"], cfg["computed_pct"]))


def test_loaded_decode_graph_replays_match_eager():
    """The Table 1 stack's decode step captured as a HIP graph gives, on
    every replay, the bits of the eager calls."""
    banner("c1-loading graph replay")
    L, N, d = 5, 1024, 512
    layers = synth.ffn_stack(7, synth.W_C1, L, N, d)
    dev_layers = [tuple(to_device_bf16(m) for m in lay) for lay in layers]
    stack = SelectInferLoadedStack(dev_layers, pct_count(30, N), pct_count(70, N), pct_count(30, N),
                                   pct_count(40, N), first=1, last=-1, max_tokens=96)
    stack.profile(dev(synth.tokens(7, synth.W_C1, 11, 64, d)),
                  dev(synth.mixture_tokens(7, synth.W_C1, 12, 32, d)))
    stack.load()
    stack.release_full_weights()
    stack.prefill(dev(synth.tokens(7, synth.W_C1, 13, 32, d)))
    X = dev(synth.tokens(7, synth.W_C1, 14, 4, d))
    eager = []
    for t in range(4):
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
        for t in range(4):
            xcur.copy_(X[t])
            g.replay()
            got = host(h)
            assert np.array_equal(got.view(np.uint32), eager[t].view(np.uint32)), (rep, t)
