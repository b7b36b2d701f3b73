"""Single SwiGLU layer, per-token top-k (Llama3.2-1B FFN shape at full size),
GPU path against the oracle, stage by stage (each stage fed the GPU's
previous output): activations within tolerance, keys / index sets
bit-exact, gathered product within tolerance."""
import numpy as np
import pytest
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from activation_sparse_decode_amd import synth
from activation_sparse_decode_amd.pipelines import SwigluSparseLayer, pct_count
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu, rel_maxabs

pytestmark = [gpu, needs_gpu]

CASES = [(1000, 264, 50), (4100, 520, 37), (8192, 2048, 50)]   # (N, d, keep %)


def make(N, d, seed=0):
    Wg = synth.weight_bf16(seed, synth.W_C0, 0, 0, synth.T_GATE, N, d)
    Wu = synth.weight_bf16(seed, synth.W_C0, 0, 0, synth.T_UP, N, d)
    WdT = synth.weight_bf16(seed, synth.W_C0, 0, 0, synth.T_DOWN, N, d)
    x = synth.tokens(seed, synth.W_C0, 0, 1, d)[0]
    return Wg, Wu, WdT, x


@pytest.mark.parametrize("keyed", [True, False])
@pytest.mark.parametrize("N,d,pct", CASES)
def test_layer_stagewise(N, d, pct, keyed):
    banner(f"c0 N={N} d={d} keep={pct}% keyed={keyed}")
    Wg, Wu, WdT, x = make(N, d)
    keep = pct_count(pct, N)
    layer = SwigluSparseLayer(dev(Wg), dev(Wu), dev(WdT), keep, keyed=keyed)
    y = torch.zeros(d, dtype=torch.float32, device="cuda")
    layer(dev(x), y)
    torch.cuda.synchronize()
    a = host(layer.a)
    assert_close(a, oracle.swiglu_acts(Wg, Wu, x), what="activations")
    assert np.array_equal(host_u32(layer.key), oracle.key_abs(a))
    idx = layer.selected()   # from the threshold pair (keyed) or the index list
    assert np.array_equal(idx, oracle.rank_range(oracle.key_abs(a), 0, keep))
    y_ref = oracle.down_gather(WdT, idx, a[idx])
    e = assert_close(host(y), y_ref, what="gathered product")
    # reported only: independent end-to-end oracle run (its own fp64 activations)
    ref = oracle.sparse_swiglu_layer(Wg, Wu, WdT, x, keep)
    overlap = np.intersect1d(ref["idx"], idx).size / max(1, keep)
    print(f"  y err {e:.2e}; end-to-end: set overlap {overlap:.4f}, "
          f"y err {rel_maxabs(host(y), ref['y']):.2e}")

    # bitwise reproducible (fixed reduction order)
    y2 = torch.zeros_like(y)
    layer(dev(x), y2)
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint32), host(y2).view(np.uint32))

    # rows that were not selected are never read: poison them with NaN
    poisoned = WdT.copy()
    skipped = np.setdiff1d(np.arange(N), idx)
    poisoned[skipped] = 0x7FC0
    y3 = torch.zeros_like(y)
    if keyed:
        B.sparse_ffn_gemv_keyed(dev(poisoned), layer.a, layer.key, B.KEY_U32, layer.thr, keep, y3,
                                workspace=layer.ws)
    else:
        B.sparse_ffn_gemv(B.OP_AXPY, dev(poisoned), None, layer.a, y3, idx=layer.idx,
                          count=layer.count, k_max=keep, workspace=layer.ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y).view(np.uint32), host(y3).view(np.uint32))


def test_full_keep_equals_dense_and_empty_selection():
    banner("c0 full keep / empty")
    N, d = 2048, 512
    Wg, Wu, WdT, x = make(N, d, seed=1)
    layer = SwigluSparseLayer(dev(Wg), dev(Wu), dev(WdT), N)
    y = torch.zeros(d, dtype=torch.float32, device="cuda")
    layer(dev(x), y)
    torch.cuda.synchronize()
    a64 = oracle.swiglu_acts(Wg, Wu, x)
    assert layer.selected().size == N
    assert_close(host(y), oracle.widen_bf16(WdT).T @ a64, what="dense")
    # keep = 0: nothing is read, y = 0; with accumulate, y is unchanged
    empty = SwigluSparseLayer(dev(Wg), dev(Wu), dev(WdT), 0)
    y0 = torch.full((d,), 3.0, dtype=torch.float32, device="cuda")
    empty(dev(x), y0)
    torch.cuda.synchronize()
    assert np.all(host(y0) == 0.0)
    y1 = torch.full((d,), 3.0, dtype=torch.float32, device="cuda")
    empty(dev(x), y1, accumulate=True)
    torch.cuda.synchronize()
    assert np.all(host(y1) == 3.0)


def test_gathered_rowops_touch_only_selected_rows():
    banner("c0 gathered row ops")
    N, d = 3000, 1024
    Wg, Wu, WdT, x = make(N, d, seed=2)
    rng = np.random.default_rng(3)
    sel = np.sort(rng.choice(N, size=777, replace=False)).astype(np.int32)
    a = torch.full((N,), 12345.0, dtype=torch.float32, device="cuda")
    key = torch.zeros(N, dtype=torch.int32, device="cuda")
    cnt = torch.tensor([sel.size], dtype=torch.int32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(Wg), dev(Wu), dev(x), a, idx=dev(sel), count=cnt,
                      k_max=sel.size, key_out=key)
    torch.cuda.synchronize()
    got = host(a)
    untouched = np.setdiff1d(np.arange(N), sel)
    assert np.all(got[untouched] == 12345.0)
    assert_close(got[sel], oracle.swiglu_acts(Wg, Wu, x, sel), what="gathered GLU")
    # k_max caps the device count
    a2 = torch.full((N,), 7.0, dtype=torch.float32, device="cuda")
    B.sparse_ffn_gemv(B.OP_GLU_SILU, dev(Wg), dev(Wu), dev(x), a2, idx=dev(sel), count=cnt, k_max=100)
    torch.cuda.synchronize()
    g2 = host(a2)
    assert np.all(g2[sel[100:]] == 7.0) and np.all(g2[sel[:100]] != 7.0)
