"""Batch-1 row operations against the oracle on both kernel shapes: rows up
to 5120 wide take the wave-per-row kernel, wider rows the workgroup-per-row
kernel.  Widths cover ragged chunk counts, the wave kernel's limit and the
wider path; 2912 rows give several rows per wave.  Cases: SwiGLU with keys
(dense, with the fused RMSNorm, and over a gathered index list that leaves
other rows untouched), plain dots added to an output, the thresholded ReLU
gate and the gated product over 32-row clusters."""
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
