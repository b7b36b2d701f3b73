"""ReLU-sparse MoE with an online cluster predictor (PowerInfer-2 guide,
"Online Predictor"): the PREDICT row op (cluster logits, and the
threshold decision sigmoid(z) > theta taken exactly on the fp32 logit),
the fused thresholded ReGLU over predicted clusters, and the stack that
predicts layer l's clusters from layer l-1's input, against the oracle
stage by stage."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import RMS_EPS, PredictedMoEStack, to_device_bf16
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]

QUANTILE = 1.2815515655446004
CLUSTER = 32


def predict(Wp, x, bias, theta, rms_eps=0.0):
    nc = Wp.shape[0]
    z = torch.full((nc,), 9.0, dtype=torch.float32, device="cuda")
    key = torch.full((nc,), -1, dtype=torch.int32, device="cuda")
    B.sparse_ffn_gemv(B.OP_PREDICT, dev(Wp), None, dev(x), z, key_out=key, tau_scale=theta,
                      aux=None if bias is None else dev(bias), rms_eps=rms_eps)
    idx = torch.full((nc,), -1, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.sparse_ffn_select(key, B.KEY_U32, 0, nc, nonzero_only=True, idx_out=idx, count_out=cnt)
    torch.cuda.synchronize()
    return host(z), host_u32(key), host(idx)[:int(host(cnt)[0])]


@pytest.mark.parametrize("nc,d", [(448, 4096), (7, 64), (1000, 520), (300, 6144)])
def test_predict_op(nc, d):
    banner(f"predict nc={nc} d={d}")
    rng = np.random.default_rng(nc + d)
    Wp = synth.weight_bf16(3, synth.W_C3, 0, 0, synth.T_PRED, nc, d)
    x = synth.tokens(3, synth.W_C3, 5, 1, d)[0]
    for bias, theta, eps in [(None, 0.45, 0.0), (rng.standard_normal(nc).astype(np.float32), 0.2, 0.0),
                             (synth.predictor_bias(nc, d, 0.45, 0.2), 0.45, RMS_EPS),
                             (None, 0.5, RMS_EPS)]:
        th32 = float(np.float32(theta))
        z, key, idx = predict(Wp, x, bias, theta, eps)
        xx = oracle.rms_normalize(x, eps) if eps > 0 else x.astype(np.float64)
        assert_close(z, oracle.predictor_logits(Wp, bias, xx), what=f"logits theta={theta}")
        exp = oracle.predicted_clusters(z.astype(np.float64), th32)   # fed the GPU's logits
        assert np.array_equal(idx, exp), theta
        nz = np.flatnonzero(key)
        assert np.array_equal(nz, exp)
        assert np.array_equal(key[nz], oracle.key_signed(z[nz]))


@pytest.mark.parametrize("theta", [0.45, 0.5, 0.3, 0.9])
def test_predict_threshold_is_exact(theta):
    """One-hot predictor rows make each logit exactly one input value; the
    inputs are the fp32 values around ln(theta / (1 - theta)), so the kernel's
    decision is checked on both sides of the threshold, bit-exact."""
    banner(f"predict threshold theta={theta}")
    th32 = float(np.float32(theta))
    t = np.float32(np.log(th32 / (1 - th32)))
    vals = [t]
    for _ in range(6):
        vals = [np.nextafter(vals[0], np.float32(-1e9), dtype=np.float32)] + vals + \
               [np.nextafter(vals[-1], np.float32(1e9), dtype=np.float32)]
    vals = np.array(vals, np.float32)
    d = 64
    x = np.zeros(d, np.float32)
    x[:vals.size] = vals
    Wp = np.zeros((vals.size, d), np.float32)
    Wp[np.arange(vals.size), np.arange(vals.size)] = 1.0
    z, key, idx = predict(synth.f32_to_bf16_bits(Wp), x, None, theta)
    assert np.array_equal(z.view(np.uint32), vals.view(np.uint32))
    assert np.array_equal(idx, oracle.predicted_clusters(vals.astype(np.float64), th32))
    assert 0 < idx.size < vals.size


@pytest.mark.parametrize("N,d", [(1024, 512), (14336, 4096), (2048, 6144)])
def test_glu_relu_op(N, d):
    banner(f"glu_relu N={N} d={d}")
    rng = np.random.default_rng(N + d)
    Wg = synth.weight_bf16(4, synth.W_C3, 0, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(4, synth.W_C3, 0, 0, synth.T_UP, N, d)
    x = synth.tokens(4, synth.W_C3, 6, 1, d)[0]
    xn = oracle.rms_normalize(x, RMS_EPS)
    tau_scale = QUANTILE * synth.WEIGHT_STD
    tau = oracle.relu_threshold(xn, QUANTILE, synth.WEIGHT_STD)
    out = torch.full((N,), 7.0, dtype=torch.float32, device="cuda")
    key = torch.zeros(N, dtype=torch.int32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GLU_RELU, dev(Wg), dev(Wu), dev(x), out, key_out=key,
                      tau_scale=tau_scale, rms_eps=RMS_EPS)
    torch.cuda.synchronize()
    ref = oracle.relu_glu_rows(Wg, Wu, xn, tau, np.arange(N))
    got = host(out)
    assert_close(got, ref, what="dense glu_relu")
    assert np.array_equal(host_u32(key), oracle.key_abs(got))
    assert 0.03 < np.mean(got != 0) < 0.2
    # over clusters only: other rows untouched
    nc = N // CLUSTER
    cl = np.sort(rng.choice(nc, size=max(1, nc // 5), replace=False)).astype(np.int32)
    out.fill_(7.0)
    B.sparse_ffn_gemv(B.OP_GLU_RELU, dev(Wg), dev(Wu), dev(x), out, idx=dev(cl),
                      count=dev(np.array([cl.size], np.int32)), k_max=cl.size, group=CLUSTER,
                      tau_scale=tau_scale, rms_eps=RMS_EPS)
    torch.cuda.synchronize()
    rows = oracle.expand_clusters(cl, CLUSTER)
    got = host(out)
    assert_close(got[rows], ref[rows], what="clustered glu_relu")
    rest = np.setdiff1d(np.arange(N), rows)
    assert np.all(got[rest] == 7.0)


def run_pred(L, E, N, d, n_tokens, check_layers, on_device_weights, seed=0):
    banner(f"c3-predictor L={L} E={E} N={N} d={d} tokens={n_tokens}")
    cfg = synth.SHAPES["c3"]
    theta, frac = cfg["pred_theta"], cfg["pred_frac"]
    th32 = float(np.float32(theta))
    nc = N // CLUSTER
    experts, preds = [], []
    for l in range(L):
        row, prow = [], []
        for e in range(E):
            if on_device_weights:
                mats = (synth.torch_weight_bf16(seed, synth.W_C3, l, e, synth.T_GATE, N, d, "cuda",
                                                cluster=CLUSTER),
                        synth.torch_weight_bf16(seed, synth.W_C3, l, e, synth.T_UP, N, d, "cuda"),
                        synth.torch_weight_bf16(seed, synth.W_C3, l, e, synth.T_DOWN, N, d, "cuda"))
                Wp = synth.torch_weight_bf16(seed, synth.W_C3, l, e, synth.T_PRED, nc, d, "cuda")
            else:
                mats = (to_device_bf16(synth.clustered_gate_bf16(seed, synth.W_C3, l, e, N, d, CLUSTER)),
                        to_device_bf16(synth.weight_bf16(seed, synth.W_C3, l, e, synth.T_UP, N, d)),
                        to_device_bf16(synth.weight_bf16(seed, synth.W_C3, l, e, synth.T_DOWN, N, d)))
                Wp = to_device_bf16(synth.weight_bf16(seed, synth.W_C3, l, e, synth.T_PRED, nc, d))
            row.append(mats)
            prow.append((Wp, dev(synth.predictor_bias(nc, d, theta, frac))))
        experts.append(row)
        preds.append(prow)
    logits = synth.router_logits(seed, synth.W_C3, L, n_tokens, E)
    X = synth.tokens(seed, synth.W_C3, 1, n_tokens, d)
    moe = PredictedMoEStack(experts, preds, CLUSTER, tau_scale=QUANTILE * synth.WEIGHT_STD,
                            theta=theta)
    ex, w = moe.route(dev(logits))
    torch.cuda.synchronize()
    w_h = host(w)
    hb = lambda t: t.cpu().numpy().view(np.uint16)  # noqa: E731
    fracs = []
    for t in range(n_tokens):
        h = dev(X[t])
        h_prev = X[t].astype(np.float32).copy()        # the predictor input of layer 0
        moe.predict(0, t, h)                           # as decode() does before layer 0
        for l in range(L):
            h_in = host(h).copy()
            got = {}

            def record(ll, tt, hh, chosen):
                got["a"] = host(moe.a).copy()
                got["z"] = host(moe.z).copy()
                got["pidx"] = host(moe.pidx).copy()
                got["pcnt"] = host(moe.pcnt).copy()
                got["chosen"] = list(chosen)

            moe.layer(l, t, h, record=record if l in check_layers else None)
            if l in check_layers:
                torch.cuda.synchronize()
                cur = l & 1
                xp = oracle.rms_normalize(h_prev, RMS_EPS)
                x = oracle.rms_normalize(h_in, RMS_EPS)
                tau = oracle.relu_threshold(x, QUANTILE, synth.WEIGHT_STD)
                y_ref = np.zeros(d)
                for j, e in enumerate(got["chosen"]):
                    Wp, bp = preds[l][e]
                    z = got["z"][cur, j]
                    assert_close(z, oracle.predictor_logits(hb(Wp), host(bp), xp),
                                 what=f"logits l={l} t={t} e={e}")
                    cl = oracle.predicted_clusters(z.astype(np.float64), th32)
                    n_c = int(got["pcnt"][cur, j])
                    assert n_c == cl.size and np.array_equal(got["pidx"][cur, j, :n_c], cl), (l, e)
                    Wg, Wu, WdT = (hb(m) for m in experts[l][e])
                    rows = oracle.expand_clusters(cl, CLUSTER)
                    a = got["a"][j][rows]
                    assert_close(a, oracle.relu_glu_rows(Wg, Wu, x, tau, rows),
                                 what=f"a l={l} t={t} e={e}")
                    y_ref += float(w_h[l * n_tokens + t, j]) * oracle.down_gather(WdT, rows, a)
                    fracs.append(n_c / nc)
                assert_close(host(h) - h_in, y_ref, what=f"h update l={l} t={t}")
            h_prev = h_in
    print(f"  predicted cluster fraction {np.mean(fracs):.3f}")
    assert 0.1 < np.mean(fracs) < 0.3


def test_small_predicted_moe():
    run_pred(L=3, E=4, N=1024, d=256, n_tokens=3, check_layers={0, 1, 2}, on_device_weights=False)


def test_full_size_predicted_moe():
    run_pred(L=32, E=8, N=14336, d=4096, n_tokens=2, check_layers={0, 1, 31},
             on_device_weights=True)


def test_moe_graph_replays_match_eager():
    """Both MoE stacks (dense gate and predictor) captured per token as HIP
    graphs give, on every replay, the bits of the eager calls (reductions in
    a fixed order, no memset nodes)."""
    from activation_sparse_decode_amd.pipelines import ReluMoEStack
    banner("c3 graph replay")
    L, E, N, d = 3, 4, 1024, 256
    nc = N // CLUSTER
    cfg = synth.SHAPES["c3"]
    experts = [[(to_device_bf16(synth.clustered_gate_bf16(6, synth.W_C3, l, e, N, d, CLUSTER)),
                 to_device_bf16(synth.weight_bf16(6, synth.W_C3, l, e, synth.T_UP, N, d)),
                 to_device_bf16(synth.weight_bf16(6, synth.W_C3, l, e, synth.T_DOWN, N, d)))
                for e in range(E)] for l in range(L)]
    preds = [[(to_device_bf16(synth.weight_bf16(6, synth.W_C3, l, e, synth.T_PRED, nc, d)),
               dev(synth.predictor_bias(nc, d, cfg["pred_theta"], cfg["pred_frac"])))
              for e in range(E)] for l in range(L)]
    T = 3
    logits = dev(synth.router_logits(6, synth.W_C3, L, T, E))
    X = dev(synth.tokens(6, synth.W_C3, 1, T, d))
    tau_scale = QUANTILE * synth.WEIGHT_STD
    for moe in (ReluMoEStack(experts, CLUSTER, tau_scale=tau_scale),
                PredictedMoEStack(experts, preds, CLUSTER, tau_scale=tau_scale,
                                  theta=cfg["pred_theta"])):
        moe.route(logits)
        eager = []
        for t in range(T):
            h = X[t].clone()
            moe.decode(h, t)
            eager.append(host(h))
        h = torch.zeros(d, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        graphs = []
        for t in range(T):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                h.copy_(X[t])
                moe.decode(h, t)
            graphs.append(g)
        for rep in range(3):
            for t in range(T):
                graphs[t].replay()
                got = host(h)                  # synchronizes between replays
                assert np.array_equal(got.view(np.uint32), eager[t].view(np.uint32)), \
                    (type(moe).__name__, rep, t)
