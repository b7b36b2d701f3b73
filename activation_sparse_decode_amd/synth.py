"""Seeded synthetic inputs for the activation-sparse decode workloads.

This module only draws random numbers and rounds the draws to the storage
dtype (fp32 -> bf16, round-to-nearest-even).  It holds none of the method's
arithmetic: no activation, ranking, selection, compaction, encoding or
contraction.  Both the GPU path (tests, bench) and the CPU oracle (tests) are
fed from here, so they see identical bytes.

Recipe (the workloads stand in for the trained models the pages measure on;
no trained weights and no dataset items are used anywhere):

* every tensor has its own stream
  ``default_rng(SeedSequence([seed, workload, layer, expert, tensor, draw]))``;
* weights are N(0, 0.02^2) drawn in fp32 and rounded RNE to bf16; they are
  stored neuron-major: row ``n`` of W_gate / W_up is neuron n's input
  weights and row ``n`` of ``W_down^T`` is neuron n's output weights;
* a decode token is ``x = z * s`` with z ~ N(0, I) and one per-channel scale
  vector ``s = exp(N(0, 1))`` per (workload, width), shared by all tokens of
  that workload (heavy-tailed input columns); a "task" is another such scale
  vector (tasks 1, 2, ... stand in for other prompt distributions, and a
  cross-task calibration set is equal blocks of tokens of tasks 0, 1, 2);
* the cluster-correlated gate of the ReLU-sparse MoE workload draws one
  centre c_k per 32-row cluster and sets row n of cluster k to
  ``0.02 * (sqrt(rho) c_k + sqrt(1 - rho) e_n)``, rho = 0.95, so the
  marginal of every entry is still N(0, 0.02^2) while neurons of a cluster
  fire together;
* router logits are N(0, 1) per (layer, token, expert);
* an (untrained) cluster predictor is a bf16 N(0, 0.02^2) matrix [clusters][d]
  with one constant bias, set so that a fraction ``frac`` of the clusters is
  predicted for an RMS-normalised input (logit ~ N(b, (0.02 sqrt(d))^2)).
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# workload ids (the five seeded workloads)
W_C0, W_C1, W_C2, W_C3, W_C4 = 0, 1, 2, 3, 4

# tensor ids
T_GATE, T_UP, T_DOWN, T_TOKEN, T_SCALE, T_ROUTER, T_QKV, T_CENTRE, T_PRED = range(9)

WEIGHT_STD = 0.02
CLUSTER_RHO = 0.95

# Workload shapes (d_model, d_ff, ...) of the models the pages evaluate.
SHAPES = {
    "c0": dict(d=2048, n=8192, keep_pct=50),                       # Llama3.2-1B FFN
    "c1": dict(d=3072, n=8192, layers=28, base_pct=20, alpha_pct=30,
               beta_pct=20, calib_tokens=512, prompt_tokens=256,
               decode_tokens=128),                                 # Llama3.2-3B FFN
    "c1_loading": dict(d=3072, n=8192, layers=28, base_pct=30, loaded_pct=70,
                       alpha_pct=30, computed_pct=40, first=5, last=-2,
                       task_tokens=512, mixture_tokens_per_task=256,
                       prompt_tokens=256, decode_tokens=128),      # SelectInfer Table 1
    "c2": dict(d=4096, qkv_out=(4096, 1024, 1024), d_ff=14336,
               top_pct=15, mid_pct=35),                            # Llama3.1-8B
    "c3": dict(d=4096, n=14336, experts=8, top_experts=2, layers=32,
               cluster=32, zero_frac_quantile=1.2815515655446004,
               decode_tokens=128, pred_theta=0.45, pred_frac=0.2),  # TurboSparse-Mixtral
    "c4": dict(d=5120, n=17408, keep_pct=40, batches=(1, 4, 8, 16)),  # Qwen-27B-like
}


def _rng(seed: int, workload: int, layer: int, expert: int, tensor: int,
         draw: int = 0) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence([seed, workload, layer, expert, tensor, draw]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the raw uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def normal_f32(seed, workload, layer, expert, tensor, shape, draw=0):
    return _rng(seed, workload, layer, expert, tensor, draw).standard_normal(
        shape, dtype=np.float32)


def weight_bf16(seed: int, workload: int, layer: int, expert: int, tensor: int,
                rows: int, cols: int) -> np.ndarray:
    """bf16 bits [rows][cols] of N(0, 0.02^2)."""
    w = normal_f32(seed, workload, layer, expert, tensor, (rows, cols))
    w *= np.float32(WEIGHT_STD)
    return f32_to_bf16_bits(w)


def clustered_gate_bf16(seed: int, workload: int, layer: int, expert: int,
                        rows: int, cols: int, cluster: int,
                        rho: float = CLUSTER_RHO) -> np.ndarray:
    """bf16 bits [rows][cols]; rows of one ``cluster``-row block share a centre."""
    assert rows % cluster == 0
    c = normal_f32(seed, workload, layer, expert, T_CENTRE, (rows // cluster, cols))
    e = normal_f32(seed, workload, layer, expert, T_GATE, (rows, cols))
    w = (np.float32(math.sqrt(rho)) * np.repeat(c, cluster, axis=0)
         + np.float32(math.sqrt(1.0 - rho)) * e)
    w *= np.float32(WEIGHT_STD)
    return f32_to_bf16_bits(w)


def channel_scale(seed: int, workload: int, d: int, task: int = 0) -> np.ndarray:
    """Per-channel lognormal(0, 1) scale, one vector per (workload, width,
    task); task 0 is the workload's own input distribution."""
    return np.exp(normal_f32(seed, workload, 0, task, T_SCALE, (d,), draw=d)).astype(np.float32)


def tokens(seed: int, workload: int, draw: int, count: int, d: int, task: int = 0) -> np.ndarray:
    """``count`` heavy-tailed tokens x = z * s, fp32 [count][d]; ``task``
    selects the scale vector (and an independent z stream for task > 0)."""
    z = normal_f32(seed, workload, 0, task, T_TOKEN, (count, d), draw=draw)
    return (z * channel_scale(seed, workload, d, task)[None, :]).astype(np.float32)


def mixture_tokens(seed: int, workload: int, draw: int, per_task: int, d: int,
                   tasks=(0, 1, 2)) -> np.ndarray:
    """A cross-task calibration set: ``per_task`` tokens of each task, in
    task blocks, fp32 [per_task * len(tasks)][d]."""
    return np.concatenate([tokens(seed, workload, draw, per_task, d, t) for t in tasks])


def predictor_bias(n_clusters: int, d: int, theta: float, frac: float) -> np.ndarray:
    """Constant fp32 bias b of a random predictor: with weights N(0, 0.02^2)
    and an input of norm sqrt(d), a logit is ~N(b, (0.02 sqrt(d))^2), and
    P(logit > ln(theta / (1 - theta))) = frac for
    b = ln(theta / (1 - theta)) - Phi^-1(1 - frac) * 0.02 * sqrt(d)."""
    from statistics import NormalDist
    b = math.log(theta / (1.0 - theta)) - NormalDist().inv_cdf(1.0 - frac) * WEIGHT_STD * math.sqrt(d)
    return np.full(n_clusters, b, dtype=np.float32)


def router_logits(seed: int, workload: int, layers: int, count: int,
                  experts: int) -> np.ndarray:
    """N(0, 1) router logits, fp32 [layers][count][experts]."""
    return normal_f32(seed, workload, 0, 0, T_ROUTER, (layers, count, experts))


def ffn_stack(seed: int, workload: int, layers: int, n: int, d: int,
              threads: int = 8) -> list:
    """[(W_gate, W_up, W_down^T)] per layer, each bf16 bits [n][d]."""
    jobs = [(l, t) for l in range(layers) for t in (T_GATE, T_UP, T_DOWN)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        mats = list(ex.map(lambda lt: weight_bf16(seed, workload, lt[0], 0, lt[1], n, d), jobs))
    return [tuple(mats[3 * l:3 * l + 3]) for l in range(layers)]


# --- device-side draws (large MoE stacks that do not fit a host round trip) ---

def torch_weight_bf16(seed: int, workload: int, layer: int, expert: int,
                      tensor: int, rows: int, cols: int, device, cluster: int = 0,
                      rho: float = CLUSTER_RHO):
    """Same recipe as the numpy weights, drawn with torch's seeded generator
    on ``device`` (used where a host draw of the whole stack is too slow).
    Returns an int16 tensor holding bf16 bits."""
    import torch
    key = (((seed * 131 + workload) * 131 + layer) * 131 + expert) * 131 + tensor
    g = torch.Generator(device=device)
    g.manual_seed(key)
    w = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    if cluster:
        g.manual_seed(key + 977)
        c = torch.randn(rows // cluster, cols, generator=g, device=device,
                        dtype=torch.float32)
        w.mul_(math.sqrt(1.0 - rho)).add_(
            c.repeat_interleave(cluster, dim=0), alpha=math.sqrt(rho))
        del c
    w.mul_(WEIGHT_STD)
    return w.to(torch.bfloat16).view(torch.int16)
