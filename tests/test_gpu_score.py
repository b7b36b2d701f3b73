"""Scores on the GPU against the oracle: Eq (1) and cluster keys bit-exact,
softmax mixing weights within tolerance."""
import numpy as np
import torch

import oracle
from activation_sparse_decode_amd import binding as B
from gpu_common import assert_close, banner, dev, gpu, host, host_u32, needs_gpu

pytestmark = [gpu, needs_gpu]


def test_eq1_bit_exact():
    banner("score eq1")
    rng = np.random.default_rng(1)
    for T, n in [(1, 100), (512, 8192), (37, 1000)]:
        a = (rng.standard_normal((T, n)) * np.exp(2 * rng.standard_normal((T, n)))).astype(np.float32)
        s = torch.zeros(n, dtype=torch.float32, device="cuda")
        B.sparse_ffn_score(B.SCORE_SUM_ABS, dev(a), s)
        got = host(s)
        assert np.array_equal(got.view(np.uint32), oracle.eq1_scores(a).view(np.uint32)), (T, n)
        # accumulate continues the same sequential sum
        B.sparse_ffn_score(B.SCORE_SUM_ABS, dev(a), s, accumulate=True)
        exp = oracle.eq1_scores(a, s0=oracle.eq1_scores(a))
        assert np.array_equal(host(s).view(np.uint32), exp.view(np.uint32))


def test_cluster_max_bit_exact():
    banner("score cluster max")
    rng = np.random.default_rng(2)
    r = np.maximum(rng.standard_normal(14336).astype(np.float32) - 1.28, 0).astype(np.float32)
    out = torch.zeros(448, dtype=torch.int32, device="cuda")
    B.sparse_ffn_score(B.SCORE_CLUSTER_MAX, dev(r), out, cluster=32)
    assert np.array_equal(host_u32(out), oracle.cluster_max_key(oracle.key_abs(r), 32))


def test_softmax_picked():
    banner("score softmax")
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((4096, 8)).astype(np.float32)
    picked = np.stack([oracle.route_top2(l)[0] for l in logits]).astype(np.int32)
    w = torch.zeros(4096, 2, dtype=torch.float32, device="cuda")
    B.sparse_ffn_score(B.SCORE_SOFTMAX_PICKED, dev(logits), w, picked=dev(picked))
    exp = np.stack([oracle.route_top2(l)[1] for l in logits])
    assert np.max(np.abs(host(w) - exp)) < 1e-6
