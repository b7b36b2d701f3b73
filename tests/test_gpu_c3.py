"""ReLU-sparse MoE stack (TurboSparse-Mixtral-like: 8 experts, 4096/14336,
32 layers at full size, top-2 routing, 32-row clusters): routing, dense
ReLU gate, cluster keys, active-cluster lists, gated up and the weighted
down accumulation, against the oracle stage by stage."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import RMS_EPS, ReluMoEStack, to_device_bf16
from gpu_common import assert_close, banner, dev, gpu, host, needs_gpu

pytestmark = [gpu, needs_gpu]

QUANTILE = 1.2815515655446004      # Phi^-1(0.9): ~10% of gate pre-activations above tau
CLUSTER = 32


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def run_moe(L, E, N, d, n_tokens, check_layers, on_device_weights, seed=0):
    banner(f"c3 L={L} E={E} N={N} d={d} tokens={n_tokens}")
    experts = []
    for l in range(L):
        row = []
        for e in range(E):
            if on_device_weights:
                Wg = synth.torch_weight_bf16(seed, synth.W_C3, l, e, synth.T_GATE, N, d, "cuda",
                                             cluster=CLUSTER)
                Wu = synth.torch_weight_bf16(seed, synth.W_C3, l, e, synth.T_UP, N, d, "cuda")
                WdT = synth.torch_weight_bf16(seed, synth.W_C3, l, e, synth.T_DOWN, N, d, "cuda")
            else:
                Wg = to_device_bf16(synth.clustered_gate_bf16(seed, synth.W_C3, l, e, N, d, CLUSTER))
                Wu = to_device_bf16(synth.weight_bf16(seed, synth.W_C3, l, e, synth.T_UP, N, d))
                WdT = to_device_bf16(synth.weight_bf16(seed, synth.W_C3, l, e, synth.T_DOWN, N, d))
            row.append((Wg, Wu, WdT))
        experts.append(row)
    logits = synth.router_logits(seed, synth.W_C3, L, n_tokens, E)
    X = synth.tokens(seed, synth.W_C3, 1, n_tokens, d)
    moe = ReluMoEStack(experts, CLUSTER, tau_scale=QUANTILE * synth.WEIGHT_STD)
    ex, w = moe.route(dev(logits))
    torch.cuda.synchronize()
    ex_h, w_h = host(ex), host(w)
    for l in range(L):
        for t in range(n_tokens):
            o_ex, o_w = oracle.route_top2(logits[l, t])
            assert np.array_equal(ex_h[l * n_tokens + t], o_ex)
            assert np.max(np.abs(w_h[l * n_tokens + t] - o_w)) < 1e-6

    stats = []
    for t in range(n_tokens):
        h = dev(X[t])
        for l in range(L):
            check = l in check_layers
            h_in = host(h).copy() if check else None
            got = {}

            def record(ll, tt, hh, chosen):
                if check:
                    torch.cuda.synchronize()
                    got["r"] = host(moe.r).copy()
                    got["cidx"] = host(moe.cidx).copy()
                    got["ccnt"] = host(moe.ccnt).copy()
                    got["a"] = host(moe.a).copy()
                    got["chosen"] = list(chosen)

            moe.layer(l, t, h, record=record)
            if not check:
                continue
            torch.cuda.synchronize()
            x = oracle.rms_normalize(h_in, RMS_EPS)
            tau = oracle.relu_threshold(x, QUANTILE, synth.WEIGHT_STD)
            y_ref = np.zeros(d)
            for j, e in enumerate(got["chosen"]):
                Wg, Wu, WdT = (host_bits(m) for m in experts[l][e])
                r = got["r"][j]
                assert_close(r, oracle.relu_gate(Wg, x, tau), what=f"r l={l} t={t} e={e}")
                clusters = oracle.active_clusters(r, CLUSTER)
                n_c = int(got["ccnt"][j])
                assert n_c == clusters.size and np.array_equal(got["cidx"][j][:n_c], clusters)
                rows = oracle.expand_clusters(clusters, CLUSTER)
                a = got["a"][j][rows]
                a_ref = r[rows].astype(np.float64) * oracle.row_dots(Wu, x, rows)
                assert_close(a, a_ref, what=f"a l={l} t={t} e={e}")
                y_ref += float(w_h[l * n_tokens + t, j]) * oracle.down_gather(WdT, rows, a)
                stats.append((np.mean(r > 0), n_c / (N // CLUSTER)))
            assert_close(host(h) - h_in, y_ref, what=f"h update l={l} t={t}")
    nz, act = np.mean([s[0] for s in stats]), np.mean([s[1] for s in stats])
    print(f"  nonzero neurons {nz:.3f}, active clusters {act:.3f}")
    assert 0.05 < nz < 0.15


def test_small_moe():
    run_moe(L=2, E=4, N=1024, d=256, n_tokens=3, check_layers={0, 1}, on_device_weights=False)


def test_full_size_moe():
    run_moe(L=32, E=8, N=14336, d=4096, n_tokens=2, check_layers={0, 31}, on_device_weights=True)


def test_gemv_lists_against_oracle():
    """The routed experts' down products as one gathered product over
    several row lists: sum_l alpha_l * sum over list l's rows of a_n W_l[n],
    added to the output; rows outside the lists are poisoned with NaN and
    must never be read; repeated calls are bitwise equal."""
    from activation_sparse_decode_amd import binding as B
    banner("c3 gemv_lists")
    rng = np.random.default_rng(21)
    N, d = 2048, 1024
    W = [synth.weight_bf16(5, synth.W_C3, 9, e, synth.T_DOWN, N, d) for e in range(3)]

    def case(group, counts, k_maxs, with_alpha):
        n_l = len(counts)
        sel = [np.sort(rng.choice(N // group, size=c, replace=False)).astype(np.int32)
               for c in counts]
        acts = [rng.standard_normal(N).astype(np.float32) for _ in range(n_l)]
        alphas = rng.uniform(0.1, 0.9, n_l).astype(np.float32) if with_alpha else np.ones(n_l, np.float32)
        Wp, y_ref = [], rng.standard_normal(d).astype(np.float64)
        y0 = y_ref.astype(np.float32)
        y_ref = y0.astype(np.float64)
        for l in range(n_l):
            used = sel[l][:min(counts[l], k_maxs[l])]
            rows = oracle.expand_clusters(used, group) if group > 1 else used
            poisoned = W[l].copy()
            keep = np.zeros(N, bool)
            keep[rows] = True
            poisoned[~keep] = 0x7FC0            # bf16 NaN in every row no list reads
            Wp.append(poisoned)
            y_ref = y_ref + float(alphas[l]) * oracle.down_gather(W[l], rows, acts[l][rows])
        out = dev(y0)
        ws = B.new_workspace(1, sum(k * group for k in k_maxs), d)
        al = [torch.tensor([a], dtype=torch.float32, device="cuda") for a in alphas]
        args = ([dev(w) for w in Wp], [dev(a) for a in acts],
                [dev(np.pad(s, (0, 1))) for s in sel],
                [torch.tensor([c], dtype=torch.int32, device="cuda") for c in counts], list(k_maxs))
        B.sparse_ffn_gemv_lists(*args, out, group=group, alphas=al if with_alpha else None,
                                accumulate=True, workspace=ws)
        torch.cuda.synchronize()
        got = host(out)
        assert np.all(np.isfinite(got)), "a row outside the lists was read"
        assert_close(got - y0, y_ref - y0, what=f"lists group={group} counts={counts}")
        out2 = dev(y0)
        B.sparse_ffn_gemv_lists(*args, out2, group=group, alphas=al if with_alpha else None,
                                accumulate=True, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(out2), got), "repeated calls differ"

    case(32, [13, 20], [N // 32, N // 32], True)          # two experts' active clusters
    case(32, [0, 17], [N // 32, N // 32], True)           # one expert with no active cluster
    case(1, [700, 31, 1200], [700, 31, 1000], False)      # single rows; k_max caps the third list
