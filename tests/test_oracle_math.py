"""Pins of the oracle's arithmetic: Eq (1), SwiGLU, the gathered product,
closed forms printed on the pages, and special cases."""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from activation_sparse_decode_amd import synth


def bf16(values):
    return synth.f32_to_bf16_bits(np.asarray(values, dtype=np.float32))


# ------------------------------------------------------------------ Eq (1)

def test_eq1_single_token_is_abs():
    a = np.array([[-1.5, 0.25, -0.0, 3.0]], dtype=np.float32)
    assert oracle.eq1_scores(a).tolist() == [1.5, 0.25, 0.0, 3.0]


def test_eq1_constant_tokens_closed_form():
    T = 512
    a = np.tile(np.array([[-0.5, 0.75, -2.0]], dtype=np.float32), (T, 1))
    assert oracle.eq1_scores(a).tolist() == [0.5 * T, 0.75 * T, 2.0 * T]


def test_eq1_is_sequential_fp32():
    # 2^24 + 1 rounds back to 2^24 in fp32 (ties to even), twice; an fp64
    # or pairwise sum would give 2^24 + 2.
    a = np.array([[2.0 ** 24], [1.0], [-1.0]], dtype=np.float32)
    assert oracle.eq1_scores(a)[0] == np.float32(2.0 ** 24)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_eq1_matches_c_float_loop():
    src = r"""
    #include <stdio.h>
    #include <stdlib.h>
    #include <math.h>
    int main(int argc, char** argv) {
      int T = atoi(argv[1]), N = atoi(argv[2]);
      FILE* f = fopen(argv[3], "rb"); FILE* g = fopen(argv[4], "wb");
      float* a = malloc(sizeof(float) * T * N); float* s = calloc(N, sizeof(float));
      if (fread(a, sizeof(float), (size_t)T * N, f) != (size_t)T * N) return 1;
      for (int t = 0; t < T; ++t) for (int n = 0; n < N; ++n) {
        volatile float v = s[n] + fabsf(a[(size_t)t * N + n]); s[n] = v; }
      fwrite(s, sizeof(float), N, g); fclose(f); fclose(g); return 0; }
    """
    rng = np.random.default_rng(7)
    T, N = 300, 257
    a = (rng.standard_normal((T, N)) * np.exp(3 * rng.standard_normal((T, N)))).astype(np.float32)
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "eq1.c")
        exe = os.path.join(d, "eq1")
        with open(c, "w") as fh:
            fh.write(src)
        subprocess.check_call(["gcc", "-O0", "-ffp-contract=off", "-o", exe, c, "-lm"])
        a.tofile(os.path.join(d, "a.bin"))
        subprocess.check_call([exe, str(T), str(N), os.path.join(d, "a.bin"), os.path.join(d, "s.bin")])
        s_c = np.fromfile(os.path.join(d, "s.bin"), dtype=np.float32)
    assert np.array_equal(s_c.view(np.uint32), oracle.eq1_scores(a).view(np.uint32))


# ------------------------------------------------------------------ SwiGLU

def test_silu_closed_forms():
    ln3 = math.log(3.0)
    s = oracle.silu(np.array([0.0, ln3, -ln3, 50.0, -800.0]))
    assert s[0] == 0.0
    assert s[1] == pytest.approx(0.75 * ln3, rel=1e-15)   # sigmoid(ln 3) = 3/4
    assert s[2] == pytest.approx(-0.25 * ln3, rel=1e-15)  # sigmoid(-ln 3) = 1/4
    assert s[3] == pytest.approx(50.0, rel=1e-15)
    assert s[4] == 0.0


def test_swiglu_one_hot_rows():
    # W_g[n] picks x_{2n}, W_u[n] picks x_{2n+1}: a_n = silu(x_{2n}) * x_{2n+1}.
    N, d = 4, 8
    Wg = np.zeros((N, d), dtype=np.float32)
    Wu = np.zeros((N, d), dtype=np.float32)
    for n in range(N):
        Wg[n, 2 * n] = 1.0
        Wu[n, 2 * n + 1] = 1.0
    x = np.array([math.log(3.0), 2.0, 0.0, 5.0, -math.log(3.0), -1.0, 1.0, 0.5], dtype=np.float32)
    a = oracle.swiglu_acts(bf16(Wg), bf16(Wu), x)
    x64 = x.astype(np.float64)
    expect = [x64[0] * 0.75 * 2.0, 0.0, x64[4] * 0.25 * -1.0, 1.0 / (1.0 + math.exp(-1.0)) * 0.5]
    # x is fp32-rounded, so ln 3 is off by ~1e-8 relative: the closed form holds to ~1e-7
    assert a.tolist() == pytest.approx(expect, rel=1e-6)


def test_row_dots_integer_bruteforce():
    rng = np.random.default_rng(11)
    W = rng.integers(-8, 9, size=(5, 7)).astype(np.float32)
    x = rng.integers(-4, 5, size=7).astype(np.float32)
    got = oracle.row_dots(bf16(W), x)
    for n in range(5):
        assert got[n] == sum(float(W[n, k]) * float(x[k]) for k in range(7))


# ------------------------------------------------------------------ gathered product

def test_down_gather_integer_bruteforce_nonsquare():
    rng = np.random.default_rng(12)
    N, d = 9, 4
    WdT = rng.integers(-8, 9, size=(N, d)).astype(np.float32)
    a = rng.integers(-3, 4, size=N).astype(np.float32)
    rows = np.array([1, 4, 8], dtype=np.int32)
    y = oracle.down_gather(bf16(WdT), rows, a[rows])
    for o in range(d):
        assert y[o] == sum(float(WdT[n, o]) * float(a[n]) for n in (1, 4, 8))


def test_full_keep_equals_dense_and_permutation_invariance():
    rng = np.random.default_rng(13)
    N, d = 64, 48
    Wg, Wu, WdT = (synth.weight_bf16(0, 9, 0, 0, t, N, d) for t in range(3))
    x = rng.standard_normal(d).astype(np.float32)
    res = oracle.sparse_swiglu_layer(Wg, Wu, WdT, x, keep=N)
    assert res["idx"].tolist() == list(range(N))
    a = res["a32"].astype(np.float64)
    dense = np.zeros(d)
    Wd64 = oracle.widen_bf16(WdT)
    for n in range(N):                       # row-by-row accumulation
        dense += a[n] * Wd64[n]
    np.testing.assert_allclose(res["y"], dense, rtol=1e-12, atol=1e-14)
    perm = rng.permutation(N)                # LeanStream: neuron order is irrelevant
    yp = oracle.down_gather(WdT[perm], np.arange(N), res["a32"][perm])
    np.testing.assert_allclose(yp, res["y"], rtol=1e-12, atol=1e-14)


def test_skipped_rows_never_contribute():
    rng = np.random.default_rng(14)
    N, d, keep = 32, 16, 10
    Wg, Wu, WdT = (synth.weight_bf16(0, 9, 1, 0, t, N, d) for t in range(3))
    x = rng.standard_normal(d).astype(np.float32)
    res = oracle.sparse_swiglu_layer(Wg, Wu, WdT, x, keep=keep)
    poisoned = WdT.copy()
    skipped = np.setdiff1d(np.arange(N), res["idx"])
    poisoned[skipped] = 0x7FC0                # bf16 NaN
    y = oracle.down_gather(poisoned, res["idx"], res["a32"][res["idx"]])
    assert np.all(np.isfinite(y))
    assert np.array_equal(y, res["y"])


def test_linearity_in_activations():
    rng = np.random.default_rng(15)
    N, d = 40, 24
    WdT = synth.weight_bf16(0, 9, 2, 0, 2, N, d)
    a = rng.standard_normal(N).astype(np.float32)
    idx = oracle.rank_range(oracle.key_abs(a), 0, 15)
    idx2 = oracle.rank_range(oracle.key_abs(2 * a), 0, 15)
    assert np.array_equal(idx, idx2)
    np.testing.assert_allclose(oracle.down_gather(WdT, idx, 2 * a[idx]),
                               2 * oracle.down_gather(WdT, idx, a[idx]), rtol=1e-14)


# ------------------------------------------------------------------ closed forms printed on the pages

def test_eq2_example():
    # SelectInfer §6.6: 2.1B x (1 - 0.7) x 0.75 x 2 bytes = 0.945 GB
    assert oracle.eq2_memory_saving(2.1e9, 0.7, 0.75, 2) == pytest.approx(0.945e9, rel=1e-12)


def test_cluster_storage_example():
    # PowerInfer-2 guide: 64 INT4 neurons x 4096 x 0.5 bytes = 131,072 bytes = 128 KB
    assert oracle.packed_bytes(64, 4096, 4) == 131072


# ------------------------------------------------------------------ FFN input normalisation

def test_rms_normalize_closed_forms():
    # [3, 4]: mean square 12.5, so the result is [3, 4] / sqrt(12.5)
    got = oracle.rms_normalize(np.array([3.0, 4.0]), 0.0)
    assert got.tolist() == pytest.approx([3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rel=1e-15)
    rng = np.random.default_rng(16)
    h = rng.standard_normal((3, 257)) * 40.0
    n = oracle.rms_normalize(h, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(n ** 2, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(oracle.rms_normalize(7.0 * h, 0.0), n, rtol=1e-14)   # scale-free
    # eps only matters for small inputs: h = 0 stays 0, tiny h is damped
    assert np.all(oracle.rms_normalize(np.zeros(5), 1e-5) == 0.0)
    assert oracle.rms_normalize(np.full(4, 1e-3), 1e-5)[0] == pytest.approx(1e-3 / math.sqrt(1e-6 + 1e-5))
