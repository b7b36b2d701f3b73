"""The fused per-neuron sparse SwiGLU (sparse_ffn_fused_swiglu) against the
oracle, stage by stage: the activations a_n it reports against
oracle.swiglu_acts over the processed set, and y against oracle.down_gather
fed those activations.  Widths cover one to eight 1 KiB chunks per row,
ragged chunk counts and the largest width (4096, where the down row is
requested late); a tall narrow case gives each wave more than 64 neurons.
Both row sources are covered: a dense (compacted) set and an index list
into the full weights, with rows outside it NaN-poisoned."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import RMS_EPS, SelectInferStack, pct_count, to_device_bf16
from gpu_common import assert_close, banner, dev, gpu, host, needs_gpu

pytestmark = [gpu, needs_gpu]

NAN_BF16 = np.uint16(0x7FC0)


def make(N, d, seed):
    Wg = synth.weight_bf16(seed, synth.W_C1, 7, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(seed, synth.W_C1, 7, 0, synth.T_UP, N, d)
    WdT = synth.weight_bf16(seed, synth.W_C1, 7, 0, synth.T_DOWN, N, d)
    x = synth.tokens(seed, synth.W_C1, 7, 2, d)
    return Wg, Wu, WdT, x[0], x[1]


def run(Wg, Wu, WdT, x, y0, *, idx=None, count=None, k_max=0, eps=0.0, accumulate=True,
        a_init=0.0):
    N, d = Wg.shape
    a = torch.full((N,), a_init, dtype=torch.float32, device="cuda")
    y = dev(y0.astype(np.float32))
    ws = B.new_workspace(1, N, d)
    B.sparse_ffn_fused_swiglu(dev(Wg), dev(Wu), dev(WdT), dev(x), y,
                              idx=None if idx is None else dev(idx.astype(np.int32)),
                              count=None if count is None else torch.tensor([count], dtype=torch.int32,
                                                                            device="cuda"),
                              k_max=k_max, rms_eps=eps, a_out=a, accumulate=accumulate,
                              workspace=ws)
    torch.cuda.synchronize()
    return host(a), host(y)


def check(Wg, Wu, WdT, x, y0, rows, a, y, eps, accumulate, what):
    xn = oracle.rms_normalize(x, eps) if eps > 0 else x
    assert_close(a[rows], oracle.swiglu_acts(Wg, Wu, xn, rows), what=f"{what} a")
    base = y0.astype(np.float64) if accumulate else 0.0
    assert_close(y - base, oracle.down_gather(WdT, rows, a[rows]), what=f"{what} y")


@pytest.mark.parametrize("d", [8, 200, 520, 1024, 2048, 2600, 3072, 3584, 4096])
def test_dense_set(d):
    N = 700
    banner(f"fused dense N={N} d={d}")
    Wg, Wu, WdT, x, y0 = make(N, d, seed=d)
    rows = np.arange(N)
    for eps, acc in ((0.0, True), (RMS_EPS, True), (RMS_EPS, False)):
        a, y = run(Wg, Wu, WdT, x, y0, eps=eps, accumulate=acc)
        check(Wg, Wu, WdT, x, y0, rows, a, y, eps, acc, f"dense d={d} eps={eps} acc={acc}")


def test_many_neurons_per_wave():
    """140000 neurons of width 8: each of the 2048 waves takes 68 neurons,
    past the 64 row numbers a wave fetches at once."""
    N, d = 140000, 8
    banner(f"fused tall N={N} d={d}")
    Wg, Wu, WdT, x, y0 = make(N, d, seed=3)
    a, y = run(Wg, Wu, WdT, x, y0, eps=RMS_EPS)
    check(Wg, Wu, WdT, x, y0, np.arange(N), a, y, RMS_EPS, True, "tall")


@pytest.mark.parametrize("d", [520, 3072, 4096])
def test_gathered_set_never_reads_skipped_rows(d):
    N = 3000
    banner(f"fused gathered N={N} d={d}")
    Wg, Wu, WdT, x, y0 = make(N, d, seed=17 + d)
    rng = np.random.default_rng(d)
    sel = np.sort(rng.choice(N, size=1203, replace=False)).astype(np.int32)
    k_max = 1500
    idx = np.concatenate([sel, rng.integers(0, N, size=k_max - sel.size)]).astype(np.int32)
    a, y = run(Wg, Wu, WdT, x, y0, idx=idx, count=sel.size, k_max=k_max, eps=RMS_EPS,
               a_init=-3.5)
    untouched = np.setdiff1d(np.arange(N), sel)
    assert np.all(a[untouched] == -3.5), "an unprocessed neuron's activation was written"
    check(Wg, Wu, WdT, x, y0, sel, a, y, RMS_EPS, True, f"gathered d={d}")

    # rows outside the set poisoned in all three matrices: bitwise the same y
    P = [np.full_like(W, NAN_BF16) for W in (Wg, Wu, WdT)]
    for Pm, W in zip(P, (Wg, Wu, WdT)):
        Pm[sel] = W[sel]
    ap, yp = run(*P, x, y0, idx=idx, count=sel.size, k_max=k_max, eps=RMS_EPS, a_init=-3.5)
    assert np.all(np.isfinite(yp)), "a skipped (NaN) row reached the output"
    assert np.array_equal(yp.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(ap.view(np.uint32), a.view(np.uint32))

    # a count above k_max is clamped to k_max
    a2, y2 = run(Wg, Wu, WdT, x, y0, idx=np.sort(idx[:k_max]), count=k_max + 500, k_max=k_max)
    rows2 = np.sort(idx[:k_max])
    assert_close(y2 - y0, oracle.down_gather(WdT, rows2, a2[rows2]), what="clamped count y")


def test_empty_sets():
    N, d = 64, 256
    banner("fused empty")
    Wg, Wu, WdT, x, y0 = make(N, d, seed=5)
    idx = np.arange(8, dtype=np.int32)
    _, y = run(Wg, Wu, WdT, x, y0, idx=idx, count=0, k_max=8)
    assert np.array_equal(y, y0.astype(np.float32))
    _, y = run(Wg, Wu, WdT, x, y0, idx=idx, count=-4, k_max=8, accumulate=False)
    assert not y.any()
    _, y = run(Wg, Wu, WdT, x, y0, idx=idx, count=5, k_max=0)
    assert np.array_equal(y, y0.astype(np.float32))
    # zero neurons, through the C entry with valid pointers (torch reports a
    # null data pointer for an empty view)
    G, xx = dev(Wg), dev(x)
    yy = dev(y0.astype(np.float32))
    ws = B.new_workspace(1, 1, d)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = B.lib().sparse_ffn_fused_swiglu(P(G), P(G), P(G), 0, d, d, P(xx), ctypes.c_float(0.0),
                                         None, None, 0, None, P(yy), 1, P(ws), ws.numel(),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, B.lib().sffn_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(host(yy), y0.astype(np.float32))


def test_records_in_place_and_reproducible():
    """One [gate | up | down] record per neuron (ld_w = 3d) gives bitwise the
    result of three separate matrices; x and y may be one buffer (the
    residual updated in place); repeated calls give the same bits."""
    N, d = 2733, 3072
    banner(f"fused records N={N} d={d}")
    Wg, Wu, WdT, x, _ = make(N, d, seed=23)
    R = torch.from_numpy(np.concatenate([Wg, Wu, WdT], axis=1).view(np.int16)).cuda()
    ws = B.new_workspace(1, N, d)
    outs = []
    for rec in (False, True, True):
        h = dev(x.astype(np.float32))
        if rec:
            B.sparse_ffn_fused_swiglu(R[:, :d], R[:, d:2 * d], R[:, 2 * d:], h, h,
                                      rms_eps=RMS_EPS, accumulate=True, workspace=ws)
        else:
            y = dev(x.astype(np.float32))
            B.sparse_ffn_fused_swiglu(dev(Wg), dev(Wu), dev(WdT), dev(x), y, rms_eps=RMS_EPS,
                                      accumulate=True, workspace=ws)
            h = y
        torch.cuda.synchronize()
        outs.append(host(h).view(np.uint32).copy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


@pytest.mark.parametrize("full", [False, True])
def test_selectinfer_stack_fused_decode(full):
    """The SelectInfer stack decoded with the fused pass, from per-prompt
    records and straight through the union index lists, layer by layer
    against the oracle (each layer fed the GPU's input to it)."""
    L, N, d = (28, 8192, 3072) if full else (3, 512, 256)
    n_calib, n_prompt = (512, 256) if full else (64, 32)
    check_layers = {0, 13, 27} if full else {0, 1, 2}
    banner(f"fused c1 stack L={L} N={N} d={d}")
    layers = synth.ffn_stack(0, synth.W_C1, L, N, d)
    dev_layers = [tuple(to_device_bf16(m) for m in lay) for lay in layers]
    stack = SelectInferStack(dev_layers, pct_count(20, N), pct_count(30, N), pct_count(20, N),
                             max_tokens=max(n_calib, n_prompt))
    stack.calibrate(dev(synth.tokens(0, synth.W_C1, 1, n_calib, d)))
    stack.prefill(dev(synth.tokens(0, synth.W_C1, 2, n_prompt, d)))
    stack.compact_records()
    U_idx, U_cnt = host(stack.U_idx), host(stack.U_cnt)
    for l in check_layers:                        # records, bit-exact
        U = U_idx[l, :U_cnt[l]]
        R = host(stack.rec[l]).view(np.uint16)
        Wg, Wu, WdT = layers[l]
        assert R.shape == (U.size, 3 * d)
        assert np.array_equal(R[:, :d], Wg[U]) and np.array_equal(R[:, d:2 * d], Wu[U])
        assert np.array_equal(R[:, 2 * d:], WdT[U])
    Xd = synth.tokens(0, synth.W_C1, 3, 2, d)
    a = torch.zeros(N, dtype=torch.float32, device="cuda")
    for t, gathered in ((0, False), (1, True)):
        h = dev(Xd[t])
        for l in range(L):
            U = U_idx[l, :U_cnt[l]]
            check = l in check_layers
            h_in = host(h).copy() if check else None
            h_two = h.clone() if check else None
            if gathered:
                stack.decode_layer_fused_gathered(l, h, a_out=a)
            else:
                stack.decode_layer_fused(l, h, a_out=a)
            if check:
                stack.decode_layer(l, h_two)      # the two-launch decode, same input
                torch.cuda.synchronize()
                Wg, Wu, WdT = layers[l]
                aa = host(a)[U] if gathered else host(a)[:U.size]
                xn = oracle.rms_normalize(h_in, RMS_EPS)
                assert_close(aa, oracle.swiglu_acts(Wg, Wu, xn, U),
                             what=f"fused a t={t} l={l} gathered={gathered}")
                assert_close(host(h) - h_in, oracle.down_gather(WdT, U, aa),
                             what=f"fused y t={t} l={l} gathered={gathered}")
                assert_close(host(h) - h_in, host(h_two) - h_in,
                             what=f"fused vs two-launch t={t} l={l}")
        torch.cuda.synchronize()
