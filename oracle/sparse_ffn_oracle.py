"""CPU oracle of the activation-sparse FFN / projection decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants) and imports
nothing from the package; it is plain numpy, fp64 wherever the pages fix no
precision, and written to be checked against the pages by eye.

Pages cited (by title and section / equation / figure):

* [SelectInfer] "SelectInfer: Selective Neuron Loading and Computation for
  On-Device LLMs" -- §3 (LLM Profiler, Eq (1)), §4 (Selective Loading),
  §5 (Selective Computation), §6.6 (Eq (2)).
* [PowerInfer-2] "PowerInfer-2: Fast 47B LLM Inference on Smartphones"
  (guide) -- "Principle 1: Neuron Cluster Decomposition" and its engine
  listing (per-cluster gate/up, silu(gate)*up, down, accumulate).
* [SpAx] "Activation Sparsity with Weight Approximation for Faster LLM
  Decoding on Offloaded Weights" -- abstract, Fig 2, Fig 3, Fig 4.
* [LeanStream] "LeanStream: A Speculate-and-Refine Streaming Framework for
  Efficient on-Device LLM Inference" -- "Permutation-Invariant Execution".
* [WiSparse] "WiSparse: Boosting LLM Inference Efficiency with Weight-Aware
  Mixed Activation Sparsity" -- abstract (weight-aware channel saliency:
  activation magnitude combined with precomputed weight norms).

Readings taken where the pages are silent: magnitude ranking |v|
everywhere; ties go to the lower index; a percentage p of N items is
floor(p*N/100); NaN ranks above +Inf and -0 equals +0; Eq (1) is a
sequential fp32 sum in token order; the dynamic set is unioned with the
static set (or, with the Table 1 knobs, dynamic neurons fill the static set
up to phi in frequency order); the 4-bit codec is min/max affine with fp16
scale/zero; the weight-aware saliency of channel j is the fp32 product
|x_j| * ||W[:, j]||_2 with the weight norm precomputed in fp32; the online
predictor's clusters are those with sigmoid(z) > theta, decided on the fp32
logit.

Parity status: every function below is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, special cases, invariants); none is unpinned.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------- scalars


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact widening)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def count_of(pct: int, n: int) -> int:
    """A ratio of ``pct`` percent of ``n`` items, as an item count.

    The pages give ratios only (SelectInfer §6.4 Table 1; SpAx Fig 2 tier
    sizes); the count is floor(pct * n / 100) in integer arithmetic."""
    return (pct * n) // 100


def key_abs(v: np.ndarray) -> np.ndarray:
    """Magnitude key of fp32 values: the fp32 bits with the sign cleared.

    Ordering these uint32 keys orders |v| (SelectInfer §2.2 ranks neurons by
    the magnitude of their activations; Eq (1) scores are sums of |a|).  -0 and
    +0 get the same key; NaN keys sort above +Inf."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    return v.view(np.uint32) & np.uint32(0x7FFFFFFF)


def key_signed(v: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 key of signed fp32 values (router logits are
    ranked by value, not magnitude)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    neg = (u >> np.uint32(31)) == 1
    return np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint32)


# ---------------------------------------------------------------- select


def rank_order(keys: np.ndarray) -> np.ndarray:
    """Indices sorted by (key descending, index ascending)."""
    keys = np.asarray(keys, dtype=np.uint32)
    n = keys.shape[0]
    return np.lexsort((np.arange(n), -keys.astype(np.int64)))


def rank_range(keys: np.ndarray, r_lo: int, r_hi: int, nonzero_only: bool = False,
               include: np.ndarray | None = None) -> np.ndarray:
    """The items at ranks [r_lo, r_hi) of the (key desc, index asc) order,
    optionally only among nonzero keys, OR-ed with ``include``; returned as
    ascending int32 indices (the compacted index list).

    Top-alpha of a token, top-beta by frequency and the top-delta base set
    (SelectInfer §4, §5) are rank ranges starting at 0; the middle tier of
    SpAx (Fig 2) is the range [k_top, k_top + k_mid)."""
    keys = np.asarray(keys, dtype=np.uint32)
    order = rank_order(keys)
    if nonzero_only:
        order = order[keys[order] != 0]
    mask = np.zeros(keys.shape[0], dtype=bool)
    mask[order[r_lo:r_hi]] = True
    if include is not None:
        mask |= np.asarray(include, dtype=bool)
    return np.flatnonzero(mask).astype(np.int32)


def cluster_max_key(keys: np.ndarray, cluster: int) -> np.ndarray:
    """kappa_c = max key over the rows [c*S_c, (c+1)*S_c) of cluster c
    (PowerInfer-2 guide, "Neuron Cluster Decomposition": a cluster is a
    block of S_c contiguous neurons)."""
    keys = np.asarray(keys, dtype=np.uint32)
    return keys.reshape(-1, cluster).max(axis=1)


def expand_clusters(clusters: np.ndarray, cluster: int) -> np.ndarray:
    """Neuron rows of the given cluster ids, ascending."""
    c = np.asarray(clusters, dtype=np.int64)
    return (c[:, None] * cluster + np.arange(cluster)[None, :]).reshape(-1).astype(np.int32)


# ---------------------------------------------------------------- Eq (1)


def eq1_scores(acts_f32: np.ndarray, s0: np.ndarray | None = None) -> np.ndarray:
    """SelectInfer §3, Eq (1): s_n = sum over tokens t of |a_n(t)|.

    Summed in fp32, one rounding per addition, tokens in order (the pages
    give no precision or order; this is the reading taken)."""
    a = np.asarray(acts_f32, dtype=np.float32)
    s = np.zeros(a.shape[1], dtype=np.float32) if s0 is None else np.array(s0, dtype=np.float32)
    for t in range(a.shape[0]):
        s = (s + np.abs(a[t])).astype(np.float32)
    return s


# ---------------------------------------------------------------- activations


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + e^-z) (the engine listing of the
    PowerInfer-2 guide applies silu to the gate and multiplies by up)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def row_dots(W_bits: np.ndarray, x: np.ndarray, rows: np.ndarray | None = None) -> np.ndarray:
    """W[n] . x for each neuron row n (fp64).  Row n of W_gate / W_up is the
    neuron's gate / up column (SelectInfer §3: a neuron is a column of the
    gate/up projections and a row of the down projection)."""
    W = W_bits if rows is None else W_bits[np.asarray(rows)]
    return widen_bf16(W) @ np.asarray(x, dtype=np.float64)


def swiglu_acts(Wg_bits, Wu_bits, x, rows=None) -> np.ndarray:
    """a_n = silu(W_g[n].x) * (W_u[n].x), fp64; the value recorded at the
    input of down_proj (SelectInfer §3)."""
    return silu(row_dots(Wg_bits, x, rows)) * row_dots(Wu_bits, x, rows)


def rms_normalize(h: np.ndarray, eps: float) -> np.ndarray:
    """Unit-gain RMSNorm of an FFN input: h / sqrt(mean(h^2) + eps), fp64.

    The pages describe the FFN alone; the stacked workloads are shaped like
    Llama3 / Mixtral blocks, which normalise the residual stream before the
    FFN.  Without it a residual stack of FFNs (each quadratic in its input)
    overflows within a few layers, so the stacks read their FFN input
    through this normalisation (the reading taken; gain 1)."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def down_gather(WdT_bits: np.ndarray, rows: np.ndarray, a_rows: np.ndarray) -> np.ndarray:
    """y = sum over selected neurons n of a_n * W_down^T[n]  (fp64).

    Only the selected rows are touched: skipped neurons contribute exactly
    zero (SelectInfer §5 computes only the selected neurons; LeanStream,
    "Permutation-Invariant Execution": the output is a sum over hidden
    neurons, so the order of the rows is irrelevant)."""
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0:
        return np.zeros(WdT_bits.shape[1], dtype=np.float64)
    return widen_bf16(WdT_bits[rows]).T @ np.asarray(a_rows, dtype=np.float64)


# ---------------------------------------------------------------- single layer (C0)


def sparse_swiglu_layer(Wg, Wu, WdT, x, keep: int):
    """One decode token through a SwiGLU FFN with per-token top-``keep``
    selection by |a| (SelectInfer §5, the per-token top-alpha step, applied
    to the token being decoded).  Returns dict(a32, keys, idx, y)."""
    a32 = swiglu_acts(Wg, Wu, x).astype(np.float32)
    keys = key_abs(a32)
    idx = rank_range(keys, 0, keep)
    y = down_gather(WdT, idx, a32[idx])
    return dict(a32=a32, keys=keys, idx=idx, y=y)


# ---------------------------------------------------------------- SelectInfer (C1)


def dense_ffn(Wg, Wu, WdT, X):
    """Dense SwiGLU FFN on tokens X [T][d]: returns (A32 [T][N], Y [T][d])."""
    X = np.asarray(X, dtype=np.float64)
    G = X @ widen_bf16(Wg).T
    U = X @ widen_bf16(Wu).T
    A32 = (silu(G) * U).astype(np.float32)
    Y = A32.astype(np.float64) @ widen_bf16(WdT)
    return A32, Y


def base_set(calib_acts_f32: np.ndarray, delta: int) -> tuple:
    """Static/base neurons: the top ``delta`` neurons by the Eq (1) score
    over the calibration tokens (SelectInfer §3 ranked neuron file, §4 top
    delta, §5 static neurons = base neurons).  Returns (s, idx)."""
    s = eq1_scores(calib_acts_f32)
    return s, rank_range(key_abs(s), 0, delta)


def dynamic_set(prompt_acts_f32: np.ndarray, alpha: int, beta: int) -> tuple:
    """SelectInfer §5 dynamic neurons: per prompt token the top ``alpha``
    neurons by |a|; count how often each neuron occurs over the prompt; keep
    the ``beta`` most frequent.  Returns (counts, idx)."""
    A = np.asarray(prompt_acts_f32, dtype=np.float32)
    counts = np.zeros(A.shape[1], dtype=np.int64)
    for t in range(A.shape[0]):
        counts[rank_range(key_abs(A[t]), 0, alpha)] += 1
    return counts, rank_range(counts.astype(np.uint32), 0, beta)


def union(*sets) -> np.ndarray:
    """Union of index sets, ascending int32 (static combined with dynamic)."""
    if not sets:
        return np.zeros(0, dtype=np.int32)
    return np.unique(np.concatenate([np.asarray(s, dtype=np.int64) for s in sets])).astype(np.int32)


def selective_loading(s_task: np.ndarray, s_model: np.ndarray, delta: int, gamma: int) -> tuple:
    """SelectInfer §4 and Fig 6: the base neurons are the top ``delta`` by
    the task-specific scores; model-specific neurons are then added in the
    order of their scores, skipping neurons already chosen, until ``gamma``
    neurons are loaded.  Returns (base, loaded), both ascending int32."""
    base = rank_range(key_abs(s_task), 0, delta)
    loaded = set(int(n) for n in base)
    for n in rank_order(key_abs(s_model)):
        if len(loaded) >= gamma:
            break
        loaded.add(int(n))
    return base, np.array(sorted(loaded), dtype=np.int32)


def loaded_positions(loaded: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Positions of neuron ids within the ascending loaded list (the resident
    weights of a selectively loaded layer hold only the loaded neurons, in
    that order).  Every id must be loaded."""
    loaded = np.asarray(loaded, dtype=np.int64)
    pos = np.searchsorted(loaded, np.asarray(ids, dtype=np.int64))
    assert np.all(pos < loaded.size) and np.array_equal(loaded[pos], ids), "id not loaded"
    return pos.astype(np.int32)


def fill_to_phi(static: np.ndarray, counts: np.ndarray, phi: int) -> np.ndarray:
    """SelectInfer §5: the static neurons are combined with dynamic neurons,
    taken in the order of their prompt frequency counts (most frequent
    first, ties to the lower index), until ``phi`` neurons are computed.
    Returns U ascending int32 (unchanged static set if it already has phi)."""
    U = set(int(n) for n in static)
    for n in rank_order(np.asarray(counts).astype(np.uint32)):
        if len(U) >= phi:
            break
        U.add(int(n))
    return np.array(sorted(U), dtype=np.int32)


def modified_layers(n_layers: int, first: int, last: int) -> range:
    """SelectInfer Table 1 layer range: layers first .. n_layers + last - 1
    (last <= 0 counts from the end; -2 skips the last two) are loaded and
    computed selectively, the others densely."""
    return range(first, n_layers + last if last <= 0 else last)


def decode_over_set(Wg, Wu, WdT, h, U):
    """A decode token at one layer computing only neurons in U: returns
    (a32 over U, y) with y = sum_{n in U} a_n W_down^T[n]."""
    a32 = swiglu_acts(Wg, Wu, h, U).astype(np.float32)
    return a32, down_gather(WdT, U, a32)


# ---------------------------------------------------------------- SpAx tiers (C2)


def tier_sets(x: np.ndarray, k_top: int, k_mid: int) -> tuple:
    """SpAx abstract / Fig 2: the k_top columns of largest |x_j| are read
    in the original format, the next k_mid from codes, the rest skipped."""
    keys = key_abs(x)
    return rank_range(keys, 0, k_top), rank_range(keys, k_top, k_top + k_mid)


def row_norms(WT_bits: np.ndarray) -> np.ndarray:
    """[WiSparse] abstract, precomputed weight norms: for W^T (row j = the
    weights of input channel j), ||W[:, j]||_2 = sqrt(sum_o W^T[j][o]^2),
    fp64."""
    w = widen_bf16(WT_bits)
    return np.sqrt(np.sum(w * w, axis=1))


def weighted_key(x: np.ndarray, norms_f32: np.ndarray) -> np.ndarray:
    """[WiSparse] abstract, weight-aware channel saliency: the activation
    magnitude times the channel's weight norm, as the fp32 product of the
    fp32 activation and the fp32 norm, keyed by magnitude."""
    prod = np.asarray(x, dtype=np.float32) * np.asarray(norms_f32, dtype=np.float32)
    return key_abs(prod.astype(np.float32))


def weighted_tier_sets(x: np.ndarray, norms_f32: np.ndarray, k_top: int, k_mid: int) -> tuple:
    """SpAx tiers (abstract, Fig 2) ranked by the [WiSparse] weight-aware
    saliency instead of |x_j| alone."""
    keys = weighted_key(x, norms_f32)
    return rank_range(keys, 0, k_top), rank_range(keys, k_top, k_top + k_mid)


def encode_4bit(WT_bits: np.ndarray, seg_rows) -> tuple:
    """SpAx Fig 3 middle tier: each input column j (a row of W^T) is coded
    with its own 4-bit uniform codes, one fp16 (scale, zero) per output
    segment (Q, K, V of Fig 4 separately).  Per column and segment:

        zero  = fp16(min w)
        scale = fp16(fp32(max w - zero) / 15)        [fp32 arithmetic]
        q     = clip(rint((w - zero) / scale), 0, 15) [fp32, half-even]
        q     = 0 where scale == 0

    Returns (scale f16 [n_in][n_seg], zero f16 [n_in][n_seg], q u8 [n_in][n_out])."""
    W = np.asarray(WT_bits, dtype=np.uint16)
    n_in, n_out = W.shape
    w32 = (W.astype(np.uint32) << np.uint32(16)).view(np.float32)
    n_seg = len(seg_rows) - 1
    scale = np.zeros((n_in, n_seg), dtype=np.float16)
    zero = np.zeros((n_in, n_seg), dtype=np.float16)
    q = np.zeros((n_in, n_out), dtype=np.uint8)
    for s in range(n_seg):
        lo, hi = seg_rows[s], seg_rows[s + 1]
        w = w32[:, lo:hi]
        z16 = w.min(axis=1).astype(np.float16)
        z32 = z16.astype(np.float32)
        rng32 = (w.max(axis=1) - z32).astype(np.float32)
        sc16 = (rng32 / np.float32(15.0)).astype(np.float32).astype(np.float16)
        sc32 = sc16.astype(np.float32)
        safe = np.where(sc32 == 0, np.float32(1.0), sc32)
        qq = np.rint(((w - z32[:, None]).astype(np.float32) / safe[:, None]).astype(np.float32))
        qq = np.clip(qq, 0, 15)
        qq[sc32 == 0, :] = 0
        q[:, lo:hi] = qq.astype(np.uint8)
        scale[:, s] = sc16
        zero[:, s] = z16
    return scale, zero, q


def decode_4bit(scale, zero, q, seg_rows) -> np.ndarray:
    """Reconstructed columns What = zero + scale * q, fp64 [n_in][n_out]."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty_like(q)
    for s in range(len(seg_rows) - 1):
        lo, hi = seg_rows[s], seg_rows[s + 1]
        out[:, lo:hi] = (zero[:, s].astype(np.float64)[:, None]
                         + scale[:, s].astype(np.float64)[:, None] * q[:, lo:hi])
    return out


def tiered_gemv(WT_bits, scale, zero, q, seg_rows, x, idx_top, idx_mid) -> np.ndarray:
    """SpAx three-tier product: y = sum_{j in top} W^T[j] x_j
    + sum_{j in mid} What^T[j] x_j; skipped columns contribute nothing."""
    x = np.asarray(x, dtype=np.float64)
    idx_top = np.asarray(idx_top, dtype=np.int64)
    idx_mid = np.asarray(idx_mid, dtype=np.int64)
    y = np.zeros(np.asarray(WT_bits).shape[1], dtype=np.float64)
    if idx_top.size:
        y += widen_bf16(WT_bits[idx_top]).T @ x[idx_top]
    if idx_mid.size:
        W_hat = decode_4bit(scale[idx_mid], zero[idx_mid], q[idx_mid], seg_rows)
        y += W_hat.T @ x[idx_mid]
    return y


# ---------------------------------------------------------------- ReLU-sparse MoE (C3)


def route_top2(logits: np.ndarray) -> tuple:
    """Top-2 experts by logit value (ties to the lower expert) and their
    mixing weights, the softmax of the two selected logits (fp64)."""
    logits = np.asarray(logits, dtype=np.float32)
    experts = rank_range(key_signed(logits), 0, 2)
    v = logits[experts].astype(np.float64)
    e = np.exp(v - v.max())
    return experts, e / e.sum()


def relu_threshold(h: np.ndarray, phi_inv_q: float, std: float) -> float:
    """tau = Phi^-1(q) * std * ||h||_2, with ``phi_inv_q`` = Phi^-1(q) (the
    standard normal quantile of q, e.g. 1.2816 for q = 0.9): the threshold
    that leaves a fraction 1-q of the gate pre-activations W_g[n].h (each
    ~ N(0, (std ||h||)^2)) above it, giving the ReLU sparsity the
    PowerInfer-2 guide describes (10-20% of neurons nonzero)."""
    return float(phi_inv_q * std * np.sqrt(np.sum(np.asarray(h, dtype=np.float64) ** 2)))


def relu_gate(Wg_bits, h, tau: float) -> np.ndarray:
    """r_n = max(W_g[n].h - tau, 0) in fp64."""
    return np.maximum(row_dots(Wg_bits, h) - tau, 0.0)


def active_clusters(r_f32: np.ndarray, cluster: int) -> np.ndarray:
    """Clusters holding at least one nonzero r_n (PowerInfer-2 guide: the
    cluster is the unit that is loaded and computed)."""
    kappa = cluster_max_key(key_abs(r_f32), cluster)
    return rank_range(kappa, 0, kappa.shape[0], nonzero_only=True)


def relu_expert(Wg, Wu, WdT, h, tau: float, cluster: int) -> dict:
    """One routed expert of the ReLU-sparse MoE at batch 1: dense gate,
    cluster activity from r, up and down only over active clusters
    (the engine listing of the PowerInfer-2 guide computes gate/up/down per
    selected cluster and accumulates)."""
    r32 = relu_gate(Wg, h, tau).astype(np.float32)
    clusters = active_clusters(r32, cluster)
    rows = expand_clusters(clusters, cluster)
    a32 = (r32[rows].astype(np.float64) * row_dots(Wu, h, rows)).astype(np.float32)
    y = down_gather(WdT, rows, a32)
    return dict(r32=r32, clusters=clusters, rows=rows, a32=a32, y=y)


def predictor_logits(Wp_bits, bias, h) -> np.ndarray:
    """PowerInfer-2 guide, "Online Predictor": the cluster logits of the
    single linear layer, z = W_pred h + b (fp64; bias may be None)."""
    z = row_dots(Wp_bits, h)
    return z if bias is None else z + np.asarray(bias, dtype=np.float64)


def predicted_clusters(z: np.ndarray, theta: float) -> np.ndarray:
    """PowerInfer-2 guide, "Online Predictor": the clusters whose predicted
    activation probability sigma(z_k) exceeds the threshold theta, ascending
    (the guide's equation writes >=, its predictor listing >; > is used:
    the two differ only where sigma(z) equals theta exactly).  sigma is
    increasing, so the test is taken as z_k > ln(theta / (1 - theta)): an
    fp64 sigmoid of a tiny z rounds to exactly 1/2 and would decide theta =
    1/2 wrongly."""
    t = np.log(theta / (1.0 - theta))
    return np.flatnonzero(np.asarray(z, dtype=np.float64) > t).astype(np.int32)


def relu_glu_rows(Wg_bits, Wu_bits, h, tau: float, rows) -> np.ndarray:
    """a_n = max(W_g[n].h - tau, 0) * (W_u[n].h) for the given rows, fp64
    (the thresholded ReGLU of the ReLU-sparse FFN, computed only where the
    predictor says the cluster is active)."""
    return np.maximum(row_dots(Wg_bits, h, rows) - tau, 0.0) * row_dots(Wu_bits, h, rows)


def predicted_expert(Wg, Wu, WdT, h, tau: float, clusters, cluster: int) -> dict:
    """One routed expert computed over predicted clusters only: gate, up
    and down read for the rows of those clusters (none of the dense gate);
    y = sum over their rows of a_n W_down^T[n]."""
    rows = expand_clusters(np.asarray(clusters, dtype=np.int64), cluster)
    a32 = relu_glu_rows(Wg, Wu, h, tau, rows).astype(np.float32)
    return dict(rows=rows, a32=a32, y=down_gather(WdT, rows, a32))


# ---------------------------------------------------------------- batched decode (C4)


def batched_union_decode(Wg, Wu, WdT, X, keep: int) -> dict:
    """Per-token top-``keep`` sets S_b, their union U, and
    Y[b] = sum_{n in S_b} a_{b,n} W_down^T[n] (a token's skipped neurons
    contribute zero even when another token selected them)."""
    X = np.asarray(X, dtype=np.float32)
    A32, S = [], []
    for b in range(X.shape[0]):
        a = swiglu_acts(Wg, Wu, X[b]).astype(np.float32)
        A32.append(a)
        S.append(rank_range(key_abs(a), 0, keep))
    U = union(*S)
    Y = np.stack([down_gather(WdT, S[b], A32[b][S[b]]) for b in range(X.shape[0])])
    return dict(A32=np.stack(A32), S=S, U=U, Y=Y)


# ---------------------------------------------------------------- byte accounting


def eq2_memory_saving(n_ffn: float, r_load: float, r_layer: float, s_bytes: float) -> float:
    """SelectInfer §6.6, Eq (2): Delta M = N_ffn (1 - r_load) r_layer s."""
    return n_ffn * (1.0 - r_load) * r_layer * s_bytes


def packed_bytes(rows: int, cols: int, bits: int) -> int:
    """Bytes of a rows x cols block stored at ``bits`` per weight (the
    PowerInfer-2 guide sizes a 64-neuron INT4 cluster at d = 4096 this way)."""
    return rows * cols * bits // 8
