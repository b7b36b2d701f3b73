"""Decode paths built from the library's entry points.

Each class owns its device buffers (allocated once, at construction) and
chains ``sparse_ffn_*`` calls on torch's current stream; selections and
counts stay on the device between calls.  The intermediate buffers are
attributes so tests can compare every stage.

* :class:`SwigluSparseLayer`   per-token top-k SwiGLU FFN at batch 1
* :class:`SelectInferStack`    SelectInfer (§3-§5): Eq (1) base set from
  calibration, per-token top-alpha / frequency top-beta from the prompt,
  union, then decode over the union in every layer
* :class:`SelectInferLoadedStack` SelectInfer with selective loading, the
  fill-to-phi computed set and the Table 1 layer range (§4, §5, §6.4)
* :class:`TieredProjection`    SpAx three-tier read (abstract, Fig 2-4)
* :class:`ReluMoEStack`        ReLU-sparse MoE with 32-row clusters
  (PowerInfer-2 guide, neuron clusters) and top-2 routing
* :class:`PredictedMoEStack`   the same stack with an online cluster predictor
  per layer and expert (PowerInfer-2 guide, "Online Predictor")
* :class:`BatchedUnionLayer`   batched decode: per-token top-k, union
  gathered once and contracted on MFMA
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B

F32, I32, U8 = torch.float32, torch.int32, torch.uint8

# The stacked workloads normalise the residual stream before each FFN, as the
# Llama3 / Mixtral blocks they are shaped like do (unit gain, eps of those
# models); the single-layer workloads feed the token to the FFN directly.
RMS_EPS = 1e-5


def to_device_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """bf16 bit patterns (numpy uint16) -> int16 device tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def pct_count(pct: int, n: int) -> int:
    """Items kept for a ratio of pct percent of n: floor(pct * n / 100)."""
    return (pct * n) // 100


def _reuse(layer, other, names) -> bool:
    """Point `layer`'s intermediate buffers at `other`'s (layers of one model
    run one after another on one stream, so they can share them)."""
    if other is None:
        return False
    for n in names:
        setattr(layer, n, getattr(other, n))
    return True


def threshold_members(keys_u32: np.ndarray, thr) -> np.ndarray:
    """Ascending indices n with key_n > T, or key_n == T and n <= I: the set a
    threshold pair (T, I) of sparse_ffn_select_threshold stands for (host
    side, for tests and reports; the keys as uint32)."""
    keys = np.asarray(keys_u32).view(np.uint32).ravel()
    T = np.uint32(int(thr[0]) & 0xFFFFFFFF)
    I = int(np.int64(thr[1]).astype(np.int32))
    n = np.arange(keys.size)
    return np.flatnonzero((keys > T) | ((keys == T) & (n <= I)))


class SwigluSparseLayer:
    """x -> a = silu(W_g x) * (W_u x) (+ keys) -> top-``keep`` by |a| ->
    y = sum over the kept neurons of a_n W_down^T[n].

    keyed (default): the selection is a threshold pair (``thr``) and the
    product forms its rows from the keys (sparse_ffn_select_threshold +
    sparse_ffn_gemv_keyed); otherwise an ascending index list and count
    (``idx``, ``count``) feed the listed product.  The selected set is the
    same either way.

    ``buffers_from``: another layer of the same shape whose intermediate
    buffers (activations, keys, selection, workspace) this one reuses,
    as the layers of a model decoded on one stream do."""

    def __init__(self, Wg, Wu, WdT, keep: int, buffers_from=None, keyed: bool = True):
        self.Wg, self.Wu, self.WdT, self.keep, self.keyed = Wg, Wu, WdT, keep, keyed
        N, d = Wg.shape
        dev = Wg.device
        if _reuse(self, buffers_from, ("a", "key", "idx", "count", "thr", "ws")):
            return
        self.a = torch.zeros(N, dtype=F32, device=dev)
        self.key = torch.zeros(N, dtype=I32, device=dev)
        self.idx = torch.zeros(max(keep, 1), dtype=I32, device=dev)
        self.count = torch.zeros(1, dtype=I32, device=dev)
        self.thr = torch.zeros(2, dtype=I32, device=dev)
        self.ws = B.new_workspace(1, keep, WdT.shape[1], device=dev)

    def __call__(self, x: torch.Tensor, y: torch.Tensor, accumulate: bool = False) -> None:
        B.sparse_ffn_gemv(B.OP_GLU_SILU, self.Wg, self.Wu, x, self.a, key_out=self.key)
        if self.keyed:
            B.sparse_ffn_select_threshold(self.key, B.KEY_U32, self.keep, self.thr)
            B.sparse_ffn_gemv_keyed(self.WdT, self.a, self.key, B.KEY_U32, self.thr, self.keep, y,
                                    accumulate=accumulate, workspace=self.ws)
            return
        B.sparse_ffn_select(self.key, B.KEY_U32, 0, self.keep, idx_out=self.idx,
                            count_out=self.count)
        B.sparse_ffn_gemv(B.OP_AXPY, self.WdT, None, self.a, y, idx=self.idx, count=self.count,
                          k_max=self.keep, accumulate=accumulate, workspace=self.ws)

    def selected(self) -> np.ndarray:
        """The last call's selected neurons, ascending (host)."""
        if self.keyed:
            return threshold_members(self.key.cpu().numpy(), self.thr.cpu().numpy())
        return self.idx.cpu().numpy()[:int(self.count.cpu()[0])]


class SelectInferStack:
    """A residual stack of SwiGLU FFN layers, h <- h + FFN_l(norm(h)), run the
    SelectInfer way: dense calibration and prefill, sparse decode over
    U_l = base_l (top delta by Eq (1)) union dynamic_l (top beta by how often
    a neuron is in a prompt token's top alpha)."""

    def __init__(self, layers, base_k: int, alpha_k: int, beta_k: int, max_tokens: int = 512,
                 rms_eps: float = RMS_EPS):
        self.layers = layers
        self.rms_eps = rms_eps
        self.L = len(layers)
        N, d = layers[0][0].shape
        self.N, self.d = N, d
        dev = layers[0][0].device
        self.base_k, self.alpha_k, self.beta_k = base_k, alpha_k, beta_k
        self.k_max = min(N, base_k + beta_k)
        self.scores = torch.zeros(self.L, N, dtype=F32, device=dev)
        self.base_mask = torch.zeros(self.L, N, dtype=U8, device=dev)
        self.freq = torch.zeros(self.L, N, dtype=I32, device=dev)
        self.U_idx = torch.zeros(self.L, N, dtype=I32, device=dev)
        self.U_cnt = torch.zeros(self.L, dtype=I32, device=dev)
        self.a = torch.zeros(self.L, N, dtype=F32, device=dev)
        self.A = torch.zeros(max_tokens, N, dtype=F32, device=dev)
        self.K = torch.zeros(max_tokens, N, dtype=I32, device=dev)
        self.ws_dense = B.new_workspace(max_tokens, N, d, device=dev)
        self.ws = B.new_workspace(1, self.k_max, d, device=dev)

    def _dense_layer(self, l: int, H: torch.Tensor, keys: bool) -> None:
        Wg, Wu, WdT = self.layers[l]
        T = H.shape[0]
        A, K = self.A[:T], self.K[:T]
        B.sparse_ffn_gemv(B.OP_GLU_SILU, Wg, Wu, H, A, key_out=K if keys else None,
                          rms_eps=self.rms_eps)

    def _dense_residual(self, l: int, H: torch.Tensor) -> None:
        T = H.shape[0]
        B.sparse_ffn_gemv(B.OP_AXPY, self.layers[l][2], None, self.A[:T], H, accumulate=True,
                          workspace=self.ws_dense)

    def calibrate(self, X: torch.Tensor, record=None) -> torch.Tensor:
        """Dense pass of calibration tokens; Eq (1) scores; base sets."""
        H = X.clone()
        self.scores.zero_()
        for l in range(self.L):
            self._dense_layer(l, H, keys=False)
            if record is not None:
                record(l, H, self.A[:H.shape[0]])
            B.sparse_ffn_score(B.SCORE_SUM_ABS, self.A[:H.shape[0]], self.scores[l])
            B.sparse_ffn_select(self.scores[l], B.KEY_ABS_F32, 0, self.base_k,
                                mask_out=self.base_mask[l])
            self._dense_residual(l, H)
        return H

    def prefill(self, X: torch.Tensor, record=None) -> torch.Tensor:
        """Dense pass of the prompt; per-token top-alpha, frequency top-beta,
        union with the base set, compacted into U_idx / U_cnt; then the
        weights of every U_l are gathered for decode (compact())."""
        H = X.clone()
        self.freq.zero_()
        T = H.shape[0]
        for l in range(self.L):
            self._dense_layer(l, H, keys=True)
            if record is not None:
                record(l, H, self.A[:T])
            B.sparse_ffn_select(self.K[:T], B.KEY_U32, 0, self.alpha_k, freq=self.freq[l])
            B.sparse_ffn_select(self.freq[l], B.KEY_U32, 0, self.beta_k,
                                include_mask=self.base_mask[l], idx_out=self.U_idx[l],
                                count_out=self.U_cnt[l:l + 1])
            self._dense_residual(l, H)
        self.compact()
        return H

    def compact(self) -> None:
        """Gather each layer's U_l weights once per prompt: gate and up rows
        side by side [|U|][2d], down rows output-major [d][|U| rounded to 8]
        (zero padded).  Reads the |U_l| counts to the host once to size the
        buffers (a per-prompt step, outside the decode loop)."""
        cnt = self.U_cnt.cpu().tolist()
        d, dev = self.d, self.U_idx.device
        self.comp = []
        for l, k in enumerate(cnt):
            Wg, Wu, WdT = self.layers[l]
            ldk = max(8, (k + 7) // 8 * 8)
            gu = torch.zeros(max(k, 1), 2 * d, dtype=torch.int16, device=dev)
            dT = torch.zeros(d, ldk, dtype=torch.int16, device=dev)
            ac = torch.zeros(ldk, dtype=F32, device=dev)
            idx = self.U_idx[l]
            B.sparse_ffn_compact(Wg, idx, k, False, gu[:, :d])
            B.sparse_ffn_compact(Wu, idx, k, False, gu[:, d:])
            B.sparse_ffn_compact(WdT, idx, k, True, dT)
            self.comp.append((gu[:k], dT, ac, k))

    def compact_records(self) -> None:
        """Gather each layer's U_l weights into one record per neuron for the
        fused decode: [gate row | up row | down row (W_down^T)], 3d bf16, so
        a layer's weights are read as one sequential stream.  A per-prompt
        step like compact() (reads the |U_l| counts to the host once)."""
        cnt = self.U_cnt.cpu().tolist()
        d, dev = self.d, self.U_idx.device
        self.rec = []
        for l, k in enumerate(cnt):
            Wg, Wu, WdT = self.layers[l]
            R = torch.zeros(max(k, 1), 3 * d, dtype=torch.int16, device=dev)
            idx = self.U_idx[l]
            B.sparse_ffn_compact(Wg, idx, k, False, R[:, :d])
            B.sparse_ffn_compact(Wu, idx, k, False, R[:, d:2 * d])
            B.sparse_ffn_compact(WdT, idx, k, False, R[:, 2 * d:])
            self.rec.append(R[:k])

    def decode_layer_fused(self, l: int, h: torch.Tensor, a_out=None) -> None:
        """Decode one layer in one pass per neuron of U_l over its records
        (gate, up, silu * mul and the down row; a second launch adds the
        workgroups' partials to the residual h in a fixed order)."""
        R, d = self.rec[l], self.d
        B.sparse_ffn_fused_swiglu(R[:, :d], R[:, d:2 * d], R[:, 2 * d:], h, h,
                                  rms_eps=self.rms_eps, a_out=a_out, accumulate=True,
                                  workspace=self.ws)

    def decode_layer_fused_gathered(self, l: int, h: torch.Tensor, a_out=None) -> None:
        """The fused pass straight from the full weights through U_l's index
        list (no compaction)."""
        Wg, Wu, WdT = self.layers[l]
        B.sparse_ffn_fused_swiglu(Wg, Wu, WdT, h, h, idx=self.U_idx[l],
                                  count=self.U_cnt[l:l + 1], k_max=self.k_max,
                                  rms_eps=self.rms_eps, a_out=a_out, accumulate=True,
                                  workspace=self.ws)

    def decode_fused(self, h: torch.Tensor) -> None:
        """One decode token through every layer with the fused pass
        (compact_records() first)."""
        for l in range(self.L):
            self.decode_layer_fused(l, h)

    def decode_layer_gathered(self, l: int, h: torch.Tensor) -> None:
        """Decode one layer straight from the full weights through U_l."""
        Wg, Wu, WdT = self.layers[l]
        idx, cnt = self.U_idx[l], self.U_cnt[l:l + 1]
        B.sparse_ffn_gemv(B.OP_GLU_SILU, Wg, Wu, h, self.a[l], idx=idx, count=cnt,
                          k_max=self.k_max, rms_eps=self.rms_eps)
        B.sparse_ffn_gemv(B.OP_AXPY, WdT, None, self.a[l], h, idx=idx, count=cnt,
                          k_max=self.k_max, accumulate=True, workspace=self.ws)

    def decode_gate_up(self, l: int, h: torch.Tensor) -> None:
        """Activations of layer l over the compacted U_l (in U_l order)."""
        gu, _, ac, k = self.comp[l]
        if k > 0:
            B.sparse_ffn_gemv(B.OP_GLU_SILU, gu[:, :self.d], gu[:, self.d:], h, ac,
                              rms_eps=self.rms_eps)

    def decode_layer(self, l: int, h: torch.Tensor) -> None:
        """Decode one layer from the compacted weights: dense gate/up over
        U_l, then one dot per output of the output-major down rows, added
        to the residual."""
        self.decode_gate_up(l, h)
        _, dT, ac, _ = self.comp[l]
        B.sparse_ffn_gemv(B.OP_DOT, dT, None, ac, h, accumulate=True)

    def decode(self, h: torch.Tensor) -> None:
        """One decode token through every layer (h is updated in place)."""
        for l in range(self.L):
            self.decode_layer(l, h)


class SelectInferLoadedStack:
    """SelectInfer with its loading and computation knobs (§4, §5, Table 1).

    Layers ``first .. L + last - 1`` are modified: only their loaded neurons
    stay resident (the top ``delta_k`` by task-specific Eq (1) scores, then
    model-specific neurons in score order until ``gamma_k``), the prompt
    ranks each token's top ``alpha_k`` among the loaded neurons, and the
    computed set is the static (base) neurons filled with the most frequent
    dynamic neurons until ``phi_k``.  The other layers are loaded and
    computed densely.  Decode streams each layer's computed set from
    per-prompt compacted buffers (dense layers: all neurons)."""

    def __init__(self, layers, delta_k: int, gamma_k: int, alpha_k: int, phi_k: int,
                 first: int = 5, last: int = -2, max_tokens: int = 512, rms_eps: float = RMS_EPS):
        self.layers = list(layers)    # full weights; profile() and load() read them
        self.rms_eps = rms_eps
        self.L = len(layers)
        N, d = layers[0][0].shape
        self.N, self.d = N, d
        dev = layers[0][0].device
        self.delta_k, self.alpha_k, self.phi_k = delta_k, alpha_k, phi_k
        self.gamma_k = min(gamma_k, N)
        assert delta_k <= self.gamma_k, "the base set must fit the loading budget"
        self.modified = set(range(first, self.L + last if last <= 0 else last))
        self.s_task = torch.zeros(self.L, N, dtype=F32, device=dev)
        self.s_model = torch.zeros(self.L, N, dtype=F32, device=dev)
        self.base_mask = torch.zeros(self.L, N, dtype=U8, device=dev)
        self.load_idx = torch.zeros(self.L, N, dtype=I32, device=dev)
        self.load_cnt = torch.zeros(self.L, dtype=I32, device=dev)
        self.s_loaded = torch.zeros(self.L, N, dtype=F32, device=dev)
        self.static_mask = torch.zeros(self.L, N, dtype=U8, device=dev)
        self.freq = torch.zeros(self.L, N, dtype=I32, device=dev)
        self.U_pos = torch.zeros(self.L, N, dtype=I32, device=dev)
        self.U_cnt = torch.zeros(self.L, dtype=I32, device=dev)
        self.A = torch.zeros(max_tokens, N, dtype=F32, device=dev)
        self.K = torch.zeros(max_tokens, N, dtype=I32, device=dev)
        self.ws_dense = B.new_workspace(max_tokens, N, d, device=dev)
        # per layer: (W_gate, W_up, W_down^T, gate|up rows side by side or None)
        self.resident = [None] * self.L

    # ---------------------------------------------------------------- offline
    def _profile_pass(self, X: torch.Tensor, scores: torch.Tensor, record=None) -> None:
        H = X.clone()
        T = H.shape[0]
        A = self.A[:T]
        for l in range(self.L):
            Wg, Wu, WdT = self.layers[l]
            B.sparse_ffn_gemv(B.OP_GLU_SILU, Wg, Wu, H, A, rms_eps=self.rms_eps)
            if record is not None:
                record(l, H, A)
            B.sparse_ffn_score(B.SCORE_SUM_ABS, A, scores[l])
            B.sparse_ffn_gemv(B.OP_AXPY, WdT, None, A, H, accumulate=True,
                              workspace=self.ws_dense)

    def profile(self, X_task: torch.Tensor, X_model: torch.Tensor, record=None) -> None:
        """Eq (1) scores of every neuron over task-specific and over
        model-specific (cross-task) calibration tokens, full model, dense."""
        self.s_task.zero_()
        self.s_model.zero_()
        self._profile_pass(X_task, self.s_task,
                           None if record is None else lambda l, H, A: record("task", l, H, A))
        self._profile_pass(X_model, self.s_model,
                           None if record is None else lambda l, H, A: record("model", l, H, A))

    def load(self) -> None:
        """Selective loading: per modified layer, base = top delta by task
        scores, then model-specific neurons until gamma; the loaded rows are
        copied into resident buffers (gate and up side by side), and the base
        set is ranked again in loaded positions (the static set of decode).
        Dense layers keep their full weights and an output-major down copy."""
        d, dev = self.d, self.s_task.device
        k = self.gamma_k
        for l in range(self.L):
            Wg, Wu, WdT = self.layers[l]
            if l not in self.modified:
                self.resident[l] = (Wg, Wu, WdT, None)
                continue
            B.sparse_ffn_select(self.s_task[l], B.KEY_ABS_F32, 0, self.delta_k,
                                mask_out=self.base_mask[l])
            B.sparse_ffn_select(self.s_model[l], B.KEY_ABS_F32, 0, k - self.delta_k,
                                include_mask=self.base_mask[l], exclude_mask=self.base_mask[l],
                                idx_out=self.load_idx[l], count_out=self.load_cnt[l:l + 1])
            gu = torch.zeros(k, 2 * d, dtype=torch.int16, device=dev)
            dn = torch.zeros(k, d, dtype=torch.int16, device=dev)
            idx = self.load_idx[l, :k]
            B.sparse_ffn_compact(Wg, idx, k, False, gu[:, :d])
            B.sparse_ffn_compact(Wu, idx, k, False, gu[:, d:])
            B.sparse_ffn_compact(WdT, idx, k, False, dn)
            self.resident[l] = (gu[:, :d], gu[:, d:], dn, gu)
            # index remap: the task scores in loaded positions, ranked again
            B.sparse_ffn_gather(self.s_task[l], idx, self.s_loaded[l, :k])
            B.sparse_ffn_select(self.s_loaded[l, :k], B.KEY_ABS_F32, 0, self.delta_k,
                                mask_out=self.static_mask[l, :k])

    def release_full_weights(self) -> None:
        """Drop the references to the full weights of the modified layers
        (only the resident buffers are used after load())."""
        for l in self.modified:
            self.layers[l] = None

    # ---------------------------------------------------------------- per prompt
    def prefill(self, X: torch.Tensor, record=None) -> torch.Tensor:
        """Prompt pass over the resident weights: modified layers compute all
        loaded neurons, rank each token's top alpha among them, count, and
        fill the static set with the most frequent neurons until phi; then
        each layer's computed set is compacted for decode."""
        H = X.clone()
        T = H.shape[0]
        k = self.gamma_k
        self.freq.zero_()
        for l in range(self.L):
            Wg, Wu, WdT, _ = self.resident[l]
            n = Wg.shape[0]
            A, K = self.A[:T, :n], self.K[:T, :n]
            sparse = l in self.modified
            B.sparse_ffn_gemv(B.OP_GLU_SILU, Wg, Wu, H, A, key_out=K if sparse else None,
                              rms_eps=self.rms_eps)
            if record is not None:
                record(l, H, A)
            if sparse:
                B.sparse_ffn_select(K, B.KEY_U32, 0, self.alpha_k, freq=self.freq[l, :k])
                B.sparse_ffn_select(self.freq[l, :k], B.KEY_U32, 0,
                                    max(0, self.phi_k - self.delta_k),
                                    include_mask=self.static_mask[l, :k],
                                    exclude_mask=self.static_mask[l, :k],
                                    idx_out=self.U_pos[l, :k], count_out=self.U_cnt[l:l + 1])
            B.sparse_ffn_gemv(B.OP_AXPY, WdT, None, A, H, accumulate=True,
                              workspace=self.ws_dense)
        self.compact()
        return H

    def compact(self) -> None:
        """Per prompt: the computed set of each modified layer gathered from
        the resident buffers (gate/up rows [|U|][2d], down output-major
        [d][|U| rounded to 8]); dense layers use all neurons.  Reads the |U|
        counts to the host once to size the buffers."""
        cnt = self.U_cnt.cpu().tolist()
        d, dev = self.d, self.s_task.device
        self.comp = []
        for l in range(self.L):
            Wg, Wu, WdT, gu_res = self.resident[l]
            if l in self.modified:
                k = cnt[l]
                idx = self.U_pos[l]
                gu = torch.zeros(max(k, 1), 2 * d, dtype=torch.int16, device=dev)
                B.sparse_ffn_compact(gu_res, idx, k, False, gu)
                W0, W1 = gu[:k, :d], gu[:k, d:]
            else:
                k = self.N
                idx = torch.arange(k, dtype=I32, device=dev)
                W0, W1 = Wg, Wu
            ldk = max(8, (k + 7) // 8 * 8)
            dT = torch.zeros(d, ldk, dtype=torch.int16, device=dev)
            B.sparse_ffn_compact(WdT, idx, k, True, dT)
            ac = torch.zeros(ldk, dtype=F32, device=dev)
            self.comp.append((W0, W1, dT, ac, k))

    # ---------------------------------------------------------------- decode
    def decode_gate_up(self, l: int, h: torch.Tensor) -> None:
        W0, W1, _, ac, k = self.comp[l]
        if k > 0:
            B.sparse_ffn_gemv(B.OP_GLU_SILU, W0, W1, h, ac, rms_eps=self.rms_eps)

    def decode_layer(self, l: int, h: torch.Tensor) -> None:
        self.decode_gate_up(l, h)
        _, _, dT, ac, _ = self.comp[l]
        B.sparse_ffn_gemv(B.OP_DOT, dT, None, ac, h, accumulate=True)

    def decode(self, h: torch.Tensor) -> None:
        for l in range(self.L):
            self.decode_layer(l, h)


class TieredProjection:
    """y = W x with the SpAx three tiers: the k_top largest |x_j| columns from
    bf16, the next k_mid from 4-bit codes, the rest skipped.

    With ``weight_aware`` the columns are ranked by the WiSparse saliency
    |x_j| * ||W[:, j]||_2 instead, the norms computed once here.
    ``keyed`` (|x| ranking only): the selection leaves the two tiers as
    threshold pairs and the product forms its columns from |x| itself, with
    no index lists.  ``buffers_from``: a projection of the same shape whose
    tier lists, counts and workspace this one reuses (projections run one
    after another)."""

    def __init__(self, Wt: torch.Tensor, seg_rows, k_top: int, k_mid: int,
                 weight_aware: bool = False, buffers_from=None, keyed: bool = True):
        self.Wt, self.seg_rows, self.k_top, self.k_mid = Wt, list(seg_rows), k_top, k_mid
        self.keyed = keyed and not weight_aware
        n_in, n_out = Wt.shape
        dev = Wt.device
        self.norms = None
        if weight_aware:
            self.norms = torch.zeros(n_in, dtype=F32, device=dev)
            B.sparse_ffn_row_norms(Wt, self.norms)
        rb = B.tier_record_bytes(n_out, len(seg_rows) - 1)
        self.rec = torch.zeros(n_in, rb, dtype=U8, device=dev)
        B.sparse_ffn_encode_tiers(Wt, self.seg_rows, self.rec)
        if _reuse(self, buffers_from, ("idx_top", "idx_mid", "cnt", "thr", "ws")):
            return
        self.idx_top = torch.zeros(max(k_top, 1), dtype=I32, device=dev)
        self.idx_mid = torch.zeros(max(k_mid, 1), dtype=I32, device=dev)
        self.cnt = torch.zeros(2, dtype=I32, device=dev)
        self.thr = torch.zeros(2, 2, dtype=I32, device=dev)    # (T, I) of the top tier, of both
        self.ws = B.new_workspace(1, k_top + k_mid, n_out, device=dev)

    def tiers(self, x: torch.Tensor):
        """Host index lists (top, mid) of the last call's tiers (tests)."""
        if not self.keyed:
            c = self.cnt.cpu().numpy()
            return (self.idx_top[:c[0]].cpu().numpy(), self.idx_mid[:c[1]].cpu().numpy())
        key = x.detach().cpu().numpy().view(np.uint32) & np.uint32(0x7FFFFFFF)
        t = self.thr.cpu().numpy()
        top = threshold_members(key, t[0])
        both = threshold_members(key, t[1])
        return top, np.setdiff1d(both, top, assume_unique=True)

    def __call__(self, x: torch.Tensor, y: torch.Tensor) -> None:
        if self.keyed:
            # one selection yields both tiers as pairs: ranks [0, k_top) and [0, k_top + k_mid)
            B.sparse_ffn_select_threshold(x, B.KEY_ABS_F32, self.k_top + self.k_mid, self.thr[1],
                                          k_top=self.k_top, thr_top_out=self.thr[0])
            B.sparse_ffn_tiered_gemv_keyed(self.Wt, self.rec, self.seg_rows, x, x, B.KEY_ABS_F32,
                                           self.thr[0], self.thr[1], self.k_top, self.k_mid, y,
                                           workspace=self.ws)
            return
        # one selection yields both tiers: ranks [0, k_top) and [k_top, k_top + k_mid)
        B.sparse_ffn_select(x, B.KEY_ABS_F32, self.k_top, self.k_top + self.k_mid,
                            idx_out=self.idx_mid, count_out=self.cnt[1:2],
                            idx_top_out=self.idx_top, count_top_out=self.cnt[0:1],
                            key_scale=self.norms)
        B.sparse_ffn_tiered_gemv(self.Wt, self.rec, self.seg_rows, x, self.idx_top, self.cnt[0:1],
                                 self.k_top, self.idx_mid, self.cnt[1:2], self.k_mid, y,
                                 workspace=self.ws)


class ReluMoEStack:
    """Residual stack of ReLU-sparse MoE FFN layers at batch 1.

    Per layer and token: top-2 experts by router logit (softmax mixing
    weights); per routed expert r = max(W_g h - tau, 0) densely, the clusters
    of 32 rows holding a nonzero r, then up and down over those clusters
    only; h <- h + sum_e w_e y_e (the expert input is norm(h))."""

    def __init__(self, experts, cluster: int, tau_scale: float, top_k: int = 2,
                 rms_eps: float = RMS_EPS):
        self.experts = experts           # [L][E] of (Wg, Wu, WdT)
        self.rms_eps = rms_eps
        self.L, self.E = len(experts), len(experts[0])
        N, d = experts[0][0][0].shape
        self.N, self.d, self.cluster, self.tau_scale, self.top_k = N, d, cluster, tau_scale, top_k
        self.nc = N // cluster
        dev = experts[0][0][0].device
        self.r = torch.zeros(top_k, N, dtype=F32, device=dev)
        self.a = torch.zeros(top_k, N, dtype=F32, device=dev)
        self.cidx = torch.zeros(top_k, self.nc, dtype=I32, device=dev)
        self.ccnt = torch.zeros(top_k, dtype=I32, device=dev)
        # cluster keys raised by the gate and reset by the select that reads them
        self.ckey = torch.zeros(top_k, self.nc, dtype=I32, device=dev)
        self.ws = B.new_workspace(1, top_k * N, d, device=dev)

    def route(self, logits: torch.Tensor):
        """logits [L][T][E] -> (experts [L*T][k] device, weights [L*T][k]
        device, experts on the host)."""
        L, T, E = logits.shape
        flat = logits.reshape(L * T, E)
        ex = torch.zeros(L * T, self.top_k, dtype=I32, device=logits.device)
        B.sparse_ffn_select(flat, B.KEY_F32, 0, self.top_k, idx_out=ex)
        w = torch.zeros(L * T, self.top_k, dtype=F32, device=logits.device)
        B.sparse_ffn_score(B.SCORE_SOFTMAX_PICKED, flat, w, picked=ex)
        self.route_idx, self.route_w, self.T = ex, w, T
        self.route_host = ex.cpu().numpy()     # expert weight pointers are chosen on the host
        return ex, w

    def layer(self, l: int, t: int, h: torch.Tensor, record=None) -> None:
        """One layer for token t.  The routed experts read the same input, so
        each step runs once for all of them: their gates in one launch, their
        active-cluster lists in one selection (a row per expert), their ups
        over those clusters in one launch, and their down products, weighted
        by the router, in one gathered product added to h."""
        row = l * self.T + t
        chosen = self.route_host[row]
        k = len(chosen)
        ex = [self.experts[l][e] for e in chosen]
        r, a = [self.r[j] for j in range(k)], [self.a[j] for j in range(k)]
        idx, cnt = [self.cidx[j] for j in range(k)], [self.ccnt[j:j + 1] for j in range(k)]
        # the gates also leave each cluster's largest |r| as its key (0: inactive)
        B.sparse_ffn_rowop_lists(B.OP_DOT_RELU_CLUSTER, [m[0] for m in ex], None, h, r,
                                 key_outs=[self.ckey[j] for j in range(k)], group=self.cluster,
                                 tau_scale=self.tau_scale, rms_eps=self.rms_eps)
        # the clusters holding a nonzero r, ascending (one call, a row per expert);
        # the keys are reset for the next layer as they are read
        B.sparse_ffn_select(self.ckey[:k], B.KEY_U32, 0, self.nc, nonzero_only=True,
                            idx_out=self.cidx[:k], count_out=self.ccnt[:k], clear_keys=True)
        B.sparse_ffn_rowop_lists(B.OP_GATED, None, [m[1] for m in ex], h, a, idxs=idx, counts=cnt,
                                 k_maxs=[self.nc] * k, group=self.cluster, auxs=r,
                                 rms_eps=self.rms_eps)
        if record is not None:
            torch.cuda.synchronize()
            record(l, t, h, chosen)
        B.sparse_ffn_gemv_lists([m[2] for m in ex], a, idx, cnt, [self.nc] * k, h,
                                group=self.cluster,
                                alphas=[self.route_w[row, j:j + 1] for j in range(k)],
                                accumulate=True, workspace=self.ws)

    def decode(self, h: torch.Tensor, t: int, record=None) -> None:
        for l in range(self.L):
            self.layer(l, t, h, record)


class PredictedMoEStack(ReluMoEStack):
    """The ReLU-sparse MoE stack with an online cluster predictor per layer
    and expert (PowerInfer-2 guide, "Online Predictor"): the clusters of
    layer l's routed experts are those with sigmoid(W_pred x + b) > theta,
    x the (normalised) FFN input of layer l - 1 (of layer 0 for layer 0).
    Each layer then reads gate, up and down rows of its predicted clusters
    only (no dense gate).  The predictors here are random: the stack shows
    the cost of the structure, not a trained predictor's accuracy."""

    def __init__(self, experts, predictors, cluster: int, tau_scale: float, theta: float,
                 top_k: int = 2, rms_eps: float = RMS_EPS):
        super().__init__(experts, cluster, tau_scale, top_k, rms_eps)
        self.predictors = predictors     # [L][E] of (W_pred bf16 [clusters][d], bias fp32 [clusters])
        self.theta = theta
        dev = experts[0][0][0].device
        nc = self.nc
        self.z = torch.zeros(2, top_k, nc, dtype=F32, device=dev)      # logits, by layer parity
        self.zkey = torch.zeros(2, top_k, nc, dtype=I32, device=dev)
        self.pidx = torch.zeros(2, top_k, nc, dtype=I32, device=dev)   # predicted clusters
        self.pcnt = torch.zeros(2, top_k, dtype=I32, device=dev)

    def predict(self, l: int, t: int, h: torch.Tensor) -> None:
        """Predicted clusters of layer l's routed experts from h (on the
        current stream) into buffer l % 2: both predictors in one launch, both
        cluster lists in one selection."""
        buf = l & 1
        chosen = self.route_host[l * self.T + t]
        k = len(chosen)
        P = [self.predictors[l][e] for e in chosen]
        B.sparse_ffn_rowop_lists(B.OP_PREDICT, [p[0] for p in P], None, h,
                                 [self.z[buf, j] for j in range(k)], auxs=[p[1] for p in P],
                                 tau_scale=self.theta,
                                 key_outs=[self.zkey[buf, j] for j in range(k)],
                                 rms_eps=self.rms_eps)
        B.sparse_ffn_select(self.zkey[buf, :k], B.KEY_U32, 0, self.nc, nonzero_only=True,
                            idx_out=self.pidx[buf, :k], count_out=self.pcnt[buf, :k])

    def layer(self, l: int, t: int, h: torch.Tensor, record=None) -> None:
        """One layer for token t: the lookahead prediction for layer l + 1
        (from this layer's input), the routed experts' ReGLU over their
        predicted clusters (one launch), then both down products, weighted
        by the router, in one gathered product added to h."""
        row = l * self.T + t
        chosen = self.route_host[row]
        k = len(chosen)
        cur = l & 1
        ex = [self.experts[l][e] for e in chosen]
        a = [self.a[j] for j in range(k)]
        idx, cnt = [self.pidx[cur, j] for j in range(k)], [self.pcnt[cur, j:j + 1] for j in range(k)]
        # The lookahead prediction is issued first on the same stream: a
        # forked stream measured slower (the graph's cross-queue waits cost
        # more than the small predictor launches).
        if l + 1 < self.L:
            self.predict(l + 1, t, h)
        B.sparse_ffn_rowop_lists(B.OP_GLU_RELU, [m[0] for m in ex], [m[1] for m in ex], h, a,
                                 idxs=idx, counts=cnt, k_maxs=[self.nc] * k, group=self.cluster,
                                 tau_scale=self.tau_scale, rms_eps=self.rms_eps)
        if record is not None:
            torch.cuda.synchronize()
            record(l, t, h, chosen)
        B.sparse_ffn_gemv_lists([m[2] for m in ex], a, idx, cnt, [self.nc] * k, h,
                                group=self.cluster,
                                alphas=[self.route_w[row, j:j + 1] for j in range(k)],
                                accumulate=True, workspace=self.ws)

    def decode(self, h: torch.Tensor, t: int, record=None) -> None:
        self.predict(0, t, h)
        for l in range(self.L):
            self.layer(l, t, h, record)


class BatchedUnionLayer:
    """A batch of tokens: per-token top-``keep`` by |a|, the union of the
    selections gathered once, each token's skipped neurons masked to zero
    (one token: its own selection is the union, passed as a threshold to the
    keyed product, or with keyed=False listed by one select; more: the
    product reads the rows some token's mask selects).
    ``buffers_from``: a layer of the same shape and batch whose intermediate
    buffers this one reuses (layers run one after another; the frequency
    counts are left at zero by every call)."""

    def __init__(self, Wg, Wu, WdT, keep: int, batch: int, buffers_from=None,
                 packed: bool = False, union_list: bool = False, keyed: bool = True):
        self.Wg, self.Wu, self.WdT, self.keep, self.batch = Wg, Wu, WdT, keep, batch
        # batch 1: the token's selection as a threshold read by the keyed
        # product (keyed), or as its listed index set
        self.keyed = keyed and batch == 1
        # batch > 1: the product forms the union from the tokens' masks
        # (SFFN_MASKED_ROWS), or with union_list the frequency counts and a
        # union select list it first
        self.union_list = union_list
        N, d = Wg.shape
        dev = Wg.device
        # packed: the batched kernels read the weights re-laid once here (gate
        # and up in row tiles, down in column panels) -- contiguous blocks
        # where the row-major layout gives 256- and 512-byte pieces of rows
        self.packed = packed and batch > 1
        if self.packed:
            self.Pg = B.pack_weights(Wg, B.LAYOUT_ROW_TILES)
            self.Pu = B.pack_weights(Wu, B.LAYOUT_ROW_TILES)
            self.Pd = B.pack_weights(WdT, B.LAYOUT_COL_PANELS)
        if _reuse(self, buffers_from, ("A", "K", "M", "F", "U", "cnt", "thr", "ws")):
            return
        self.A = torch.zeros(batch, N, dtype=F32, device=dev)
        self.K = torch.zeros(batch, N, dtype=I32, device=dev)
        # token masks with a row stride of a multiple of 16 bytes (the masked
        # product reads them 16 bytes at a time)
        self.M = torch.zeros(batch, (N + 15) // 16 * 16, dtype=U8, device=dev)[:, :N]
        self.F = torch.zeros(N, dtype=I32, device=dev)
        self.U = torch.zeros(N, dtype=I32, device=dev)
        self.cnt = torch.zeros(1, dtype=I32, device=dev)
        self.thr = torch.zeros(2, dtype=I32, device=dev)
        self.ws = B.new_workspace(batch, N, d, device=dev)

    def __call__(self, X: torch.Tensor, Y: torch.Tensor) -> None:
        N = self.Wg.shape[0]
        Wg, Wu, WdT = (self.Pg, self.Pu, self.Pd) if self.packed else (self.Wg, self.Wu, self.WdT)
        # the workspace lets the batched gate/up split its last tiles along K
        B.sparse_ffn_gemv(B.OP_GLU_SILU, Wg, Wu, X, self.A, key_out=self.K, workspace=self.ws)
        if self.keyed:
            # one token: the union is the token's own set; the product reads
            # the rows the token's threshold selects, with no list
            B.sparse_ffn_select_threshold(self.K, B.KEY_U32, self.keep, self.thr)
            B.sparse_ffn_gemv_keyed(WdT, self.A, self.K, B.KEY_U32, self.thr, self.keep, Y,
                                    workspace=self.ws)
            return
        if self.batch == 1:
            # one token: the union is the token's own set, so its ascending
            # list comes straight from the token's select (the frequency
            # counts and the union select would return the same list), and
            # every listed row is the token's (no mask in the product)
            B.sparse_ffn_select(self.K, B.KEY_U32, 0, self.keep, mask_out=self.M, idx_out=self.U,
                                count_out=self.cnt)
            B.sparse_ffn_gemv(B.OP_AXPY, WdT, None, self.A, Y, idx=self.U, count=self.cnt,
                              k_max=N, workspace=self.ws)
            return
        if not self.union_list:
            B.sparse_ffn_select(self.K, B.KEY_U32, 0, self.keep, mask_out=self.M)
            B.sparse_ffn_gemv(B.OP_AXPY | B.MASKED_ROWS, WdT, None, self.A, Y, row_mask=self.M,
                              workspace=self.ws)
            return
        # F starts at zero (allocation) and the union select resets it as it
        # reads it, ready for the next batch's counts
        B.sparse_ffn_select(self.K, B.KEY_U32, 0, self.keep, mask_out=self.M, freq=self.F)
        B.sparse_ffn_select(self.F, B.KEY_U32, 0, N, nonzero_only=True, idx_out=self.U,
                            count_out=self.cnt, clear_keys=True)
        B.sparse_ffn_gemv(B.OP_AXPY, WdT, None, self.A, Y, idx=self.U, count=self.cnt,
                          k_max=N, row_mask=self.M, workspace=self.ws)
