/*
 * sparse_ffn.h -- C ABI of the MI355X (gfx950) activation-sparse FFN /
 * projection decode library (libsparse_ffn.so).
 *
 * The library implements the decode hot path shared by these pages:
 *   [SelectInfer] "SelectInfer: Selective Neuron Loading and Computation for
 *                 On-Device LLMs"
 *   [PowerInfer-2] "PowerInfer-2: Fast 47B LLM Inference on Smartphones" (guide)
 *   [SpAx]        "Activation Sparsity with Weight Approximation for Faster
 *                 LLM Decoding on Offloaded Weights"
 *   [LeanStream]  "LeanStream: A Speculate-and-Refine Streaming Framework for
 *                 Efficient on-Device LLM Inference"
 *   [WiSparse]    "WiSparse: Boosting LLM Inference Efficiency with
 *                 Weight-Aware Mixed Activation Sparsity" (abstract)
 * namely: compute activations, score / rank them by magnitude, select rank
 * ranges, compact the selection into ascending index lists, and read only
 * the selected weight rows in a gathered matrix-vector product (plus the
 * SpAx three-tier read).
 *
 * Conventions shared by every call
 *  - Every array pointer is a DEVICE pointer owned by the caller.  Nothing
 *    here allocates, frees or synchronises; nothing reads device memory on
 *    the host.  All work is enqueued on `stream` (a hipStream_t; NULL is the
 *    null stream).  Counts produced by one call are read on the device by
 *    the next, so select -> gemv chains never round-trip through the host.
 *  - Weights are bf16 bit patterns (uint16_t), stored neuron-major: row n of
 *    W_gate / W_up holds neuron n's input weights, row n of W_down^T holds
 *    its output weights; [SelectInfer] §3 identifies a neuron with a column
 *    of gate/up and a row of down.  Row pitch `ld_w` is in elements.
 *  - Activations and outputs are fp32; keys are uint32; indices and counts
 *    are int32.  2-D arrays are row-major with the stated leading dimension
 *    (elements).
 *  - Arguments are checked before anything is launched.  On a bad argument a
 *    call returns SFFN_EINVAL / SFFN_EUNSUPPORTED / SFFN_EWORKSPACE, launches
 *    nothing, and sffn_last_error() describes the problem.  A failed launch
 *    returns SFFN_EHIP with the HIP error text.  No C++ exception crosses the
 *    ABI.
 *  - Device-side preconditions that cannot be checked on the host:
 *    0 <= idx[i] < n_rows / group, indices in a list are distinct, and
 *    counts are >= 0; kernels process min(*count, k_max) entries.
 *    Checked mode, for debugging: with the environment variable
 *    SFFN_DEBUG_CHECKS set to anything but "0" (read at every call), a call
 *    that takes device index lists (gemv, gemv_noalloc, gemv_lists,
 *    rowop_lists, fused_swiglu, tiered_gemv, compact) waits for its stream,
 *    reads the counts and lists on the host and checks these preconditions
 *    before launching; a violation returns SFFN_EINVAL naming the entry and
 *    launches nothing.  That mode synchronises and reads device memory, so
 *    it is not for use under graph capture or in timed runs.
 *  - Calls that take a workspace use it as scratch for split-K partials and
 *    packed operands; it needs no initialisation.  One workspace must not be
 *    used by two calls that may run at the same time.
 */
#ifndef SPARSE_FFN_H
#define SPARSE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SFFN_OK = 0,
    SFFN_EINVAL = 1,        /* bad argument (null, misaligned, out of range) */
    SFFN_EUNSUPPORTED = 2,  /* valid but outside what the kernels handle      */
    SFFN_EWORKSPACE = 3,    /* workspace missing or too small                 */
    SFFN_EHIP = 4           /* the HIP runtime reported an error              */
} sffn_status;

/* How select turns its input into an ordering key (uint32, larger = earlier). */
typedef enum {
    SFFN_KEY_ABS_F32 = 0,   /* fp32 input, key = bits & 0x7FFFFFFF: orders |v|;
                               -0 == +0; NaN above +Inf ([SelectInfer] §2.2 ranks
                               neurons by activation magnitude)                 */
    SFFN_KEY_U32 = 1,       /* uint32 input used as the key (frequency counts)  */
    SFFN_KEY_F32 = 2        /* fp32 input ordered by signed value (router logits) */
} sffn_key_type;

typedef enum {
    SFFN_SCORE_SUM_ABS = 0,        /* [SelectInfer] §3 Eq (1): s_n (+)= sum_t |a_n(t)|,
                                      fp32, one rounding per add, t ascending      */
    SFFN_SCORE_CLUSTER_MAX = 1,    /* kappa_c = max over the `cluster` rows of
                                      cluster c of the magnitude key (exact)       */
    SFFN_SCORE_SOFTMAX_PICKED = 2  /* w_j = softmax over the k picked entries      */
} sffn_score_mode;

typedef enum {
    SFFN_OP_GLU_SILU = 0,   /* out_n = silu(W0[n].x) * (W1[n].x)        (SwiGLU)  */
    SFFN_OP_DOT_RELU = 1,   /* out_n = max(W0[n].x - tau_scale*||x||_2, 0) (ReGLU gate) */
    SFFN_OP_GATED = 2,      /* out_n = aux_n * (W1[n].x)                 (ReGLU up) */
    SFFN_OP_AXPY = 3,       /* y (+)= alpha * sum_n m_n in_n W0[n][:]    (down)     */
    SFFN_OP_DOT = 4,        /* out_n = W0[n].x   (down over compacted, output-major
                               weights: one dot per output)                      */
    SFFN_OP_GLU_RELU = 5,   /* out_n = max(W0[n].x - tau_scale*||x||_2, 0) * (W1[n].x)
                               (thresholded ReGLU, both matrices in one pass)    */
    SFFN_OP_PREDICT = 6,    /* out_n = W0[n].x + aux_n (cluster logits of the online
                               predictor); key nonzero iff sigmoid(out_n) > theta */
    SFFN_OP_DOT_RELU_CLUSTER = 7 /* out_n as DOT_RELU; key_out holds cluster keys:
                               key_out[c] = max(key_out[c], bits(out_n) & 0x7FFFFFFF)
                               over the nonzero rows n of cluster c = n / group   */
} sffn_gemv_op;

/* Flag OR-ed into a sparse_ffn_gemv op: W0 / W1 are in the packed layout of
   the batched (batch > 1) kernels, built by sparse_ffn_pack_weights: the
   row-tile layout for the row ops (GLU_SILU, DOT_RELU, GATED, DOT), the
   column-panel layout for AXPY.  Same rows processed, same arithmetic in the
   same order: results are bitwise those of the row-major weights. */
#define SFFN_PACKED 0x100

/* Flag OR-ed into SFFN_OP_AXPY at batch > 1 with idx NULL and a row_mask:
   only the rows whose mask is nonzero for some token of the batch are read
   -- the union of the tokens' selections ([SelectInfer] §5; [LeanStream]
   "Permutation-Invariant Execution": the union read once as one dense
   block) formed inside the product, in index order, with no index list or
   count.  The result is that of the union's index list (up to the order
   of fp32 additions).  Needs row_mask 16-byte aligned and ld_mask % 16 == 0
   (EINVAL), batch > 1 (EUNSUPPORTED). */
#define SFFN_MASKED_ROWS 0x200

/* Packed weight layouts (sparse_ffn_pack_weights). */
typedef enum {
    /* [ceil(n/16)][d/128][16][128]: element (r, k) at ((r/16)*(d/128) + k/128)
       * 2048 + (r%16)*128 + k%128; rows past n are zero.  A batched row op
       reads 16 rows x 128 k of one tile as one contiguous 4 KB block. */
    SFFN_LAYOUT_ROW_TILES = 1,
    /* [d/256][n][256]: element (r, o) at (o/256)*n*256 + r*256 + o%256.  The
       batched AXPY reads a row's 256 outputs of one panel as one contiguous
       512-byte piece, the rows of a panel back to back. */
    SFFN_LAYOUT_COL_PANELS = 2
} sffn_layout;

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* sffn_last_error(void);

/* ABI revision of this header (bumped on any change of a signature or of what
   a call computes, e.g. a new op or option). */
int sffn_abi_version(void);
#define SFFN_ABI_VERSION 17

/* Bytes of workspace sparse_ffn_gemv / sparse_ffn_tiered_gemv need for a
 * product with `batch` tokens, up to `n_rows` gathered rows (after cluster
 * expansion) and `d_out` outputs per token. */
size_t sparse_ffn_workspace_size(int batch, int n_rows, int d_out);

/*
 * sparse_ffn_score -- per-neuron or per-cluster scores.
 *  in   : fp32 [T][ld] (ld >= n).
 *  SUM_ABS:  out = fp32 [n]; s_n = (accumulate ? s_n : 0) + |in[0][n]| + ... +
 *            |in[T-1][n]|, added left to right in fp32 ([SelectInfer] §3,
 *            Eq (1); the offline profiler's neuron score).
 *  CLUSTER_MAX: out = uint32 [T][n / cluster]; out[t][c] = max over rows
 *            c*cluster .. c*cluster+cluster-1 of (bits(in[t][row]) & 0x7FFFFFFF)
 *            ([PowerInfer-2], "Neuron Cluster Decomposition": a cluster is a
 *            block of S_c contiguous neurons); n % cluster == 0.
 *  SOFTMAX_PICKED: picked = int32 [T][k] column indices (< n), out = fp32
 *            [T][k]; out[t][j] = exp(in[t][p_j] - m) / sum_j' exp(in[t][p_j'] - m),
 *            m = max_j in[t][p_j] (mixing weights of the routed experts).
 *  `picked`/`k` are ignored by the other modes; `cluster`/`accumulate` are
 *  ignored where they do not apply.
 */
sffn_status sparse_ffn_score(int mode, const float* in, int T, int n, int ld,
                             int cluster, int accumulate,
                             const int32_t* picked, int k,
                             void* out, void* stream);

/*
 * sparse_ffn_select -- rank-range selection and compaction, one row at a time.
 * For each row r < rows, the n entries of keys + r*ld are ordered by (key
 * descending, index ascending) and the entries at ranks [r_lo, r_hi) are
 * selected.  Top-k ([SelectInfer] §5 per-token top alpha and top beta by
 * frequency, §4 top delta) is the range [0, k); the SpAx middle tier (Fig 2)
 * is [k_top, k_top + k_mid), and the same call can return the top tier
 * [0, k_top) as a second list.
 *  cluster      : entry c is the block of `cluster` contiguous values
 *                 keys[c*cluster .. c*cluster+cluster-1] and its key is the
 *                 largest key of the block ([PowerInfer-2] "Neuron Cluster
 *                 Decomposition": a cluster is selected as a unit); 1 for
 *                 single values.  ld >= n * cluster; with cluster > 1,
 *                 n <= 4096 and n * cluster <= 2^30 (else
 *                 SFFN_EUNSUPPORTED).  Value i belongs to cluster
 *                 i / cluster exactly, for any cluster size.
 *  key_scale    : nullable fp32 [n]; with SFFN_KEY_ABS_F32 keys and
 *                 cluster == 1 only.  The key of entry j becomes the magnitude
 *                 key of the fp32 product keys[r][j] * key_scale[j]: the
 *                 weight-aware channel saliency of [WiSparse] (activation
 *                 magnitude times a precomputed weight norm, e.g. from
 *                 sparse_ffn_row_norms of the projection's W^T).
 *  nonzero_only : only entries with a nonzero key take part (ranks count
 *                 among them); not allowed with SFFN_KEY_F32.
 *  include_mask : nullable uint8 [n]; nonzero entries are OR-ed into every
 *                 row's selection (union with a static set, [SelectInfer] §5).
 *  exclude_mask : nullable uint8 [n]; nonzero entries take no part in the
 *                 ranking (ranks count among the others).  With the same
 *                 mask as include_mask and [0, k) the result is the set plus
 *                 the k best-ranked entries outside it: the secondary neurons
 *                 added to the base neurons until the loading budget is met
 *                 ([SelectInfer] §4, Fig 6), and the dynamic neurons added to
 *                 the static ones until the computed fraction is reached
 *                 (§5).  An entry in both masks is selected through the
 *                 include mask only (not in idx_top_out).
 *  mask_out     : nullable uint8 [rows][ld_mask], 1 = selected, 0 otherwise.
 *  idx_out      : nullable int32 [rows][ld_idx]: selected indices, ascending.
 *                 ld_idx >= n if include_mask is set, else >= r_hi - r_lo.
 *  count_out    : nullable int32 [rows]: number selected.
 *  idx_top_out  : nullable int32 [rows][ld_idx_top]: the entries at ranks
 *                 [0, r_lo), ascending (ld_idx_top >= r_lo); count_top_out
 *                 nullable int32 [rows] their number.  Not affected by
 *                 include_mask.
 *  freq_inout   : nullable uint32 [n]: += 1 for each row that selects the
 *                 entry (the frequency count of [SelectInfer] §5).
 *  clear_keys   : nonzero: each row's keys[r][0..n) are set to 0 once read
 *                 (cluster == 1, no key_scale), so a frequency count can be
 *                 consumed and reset for its next accumulation in one pass
 *                 (keys is then written: it must not be read-only memory).
 * Limits: 1 <= n <= 32768, 0 <= r_lo <= r_hi, r_hi may exceed the number of
 * eligible entries (then it is clipped).  The result is unique: bit-exact.
 */
sffn_status sparse_ffn_select(const void* keys, int key_type, const float* key_scale,
                              int rows, int n, int ld,
                              int cluster, int r_lo, int r_hi, int nonzero_only,
                              const uint8_t* include_mask,
                              const uint8_t* exclude_mask,
                              uint8_t* mask_out, int ld_mask,
                              int32_t* idx_out, int ld_idx,
                              int32_t* count_out,
                              int32_t* idx_top_out, int ld_idx_top,
                              int32_t* count_top_out,
                              uint32_t* freq_inout,
                              int clear_keys,
                              void* stream);

/*
 * sparse_ffn_select_threshold -- the top-k rank range [0, k) of each row as
 * a threshold instead of a list ([SelectInfer] §5: per token, the k neurons
 * with the largest activation magnitudes).  The n entries of keys + r*ld
 * (row r < rows) are ordered by (key descending, index ascending), as
 * sparse_ffn_select orders them, and thr_out[2r], thr_out[2r+1] receive
 * (T, I): entry j is among the first k iff key_j > T, or key_j == T and
 * j <= I (I read as int32).  k = 0 gives (0xFFFFFFFF, -1), nothing; k >= n
 * gives (0, 0x7FFFFFFF), everything.  The set is that of sparse_ffn_select
 * with r_lo = 0, r_hi = k and no masks, entry for entry; no index list,
 * count or mask is written -- a consumer such as sparse_ffn_gemv_keyed
 * applies the test to the keys itself.  With k_top > 0, thr_top_out[2r],
 * thr_top_out[2r+1] receive the pair of [0, k_top) as well, from the same
 * pass (the SpAx top tier; the middle tier [k_top, k) is the set of thr_out
 * less that of thr_top_out).  With k_top = 0 a non-null thr_top_out
 * receives the empty pair.
 *  keys        : [rows][ld] in key_type's representation (ld >= n), 4-byte
 *                aligned.
 *  thr_out     : uint32 [rows][2], 8-byte aligned.
 *  thr_top_out : nullable uint32 [rows][2], 8-byte aligned; required when
 *                k_top > 0.
 * Limits: 1 <= n <= 32768 (EUNSUPPORTED outside), 0 <= k_top <= k,
 * rows >= 0.
 */
sffn_status sparse_ffn_select_threshold(const void* keys, int key_type, int rows, int n, int ld,
                                        int k_top, int k, uint32_t* thr_top_out,
                                        uint32_t* thr_out, void* stream);

/*
 * sparse_ffn_gemv -- activations and gathered products over weight rows.
 * Rows processed: all n_rows rows when idx is NULL; otherwise, for
 * i < min(*count, k_max) and g < group, row idx[i]*group + g (a cluster of
 * `group` contiguous rows per index, [PowerInfer-2] "Neuron Cluster
 * Decomposition"; group = 1 for single neurons).  Skipped rows are never
 * read ([SelectInfer] §5 computes only the selected neurons).
 *
 * Row ops (GLU_SILU, DOT_RELU, GATED, DOT): W0, W1 are bf16 [n_rows][ld_w]
 *  with rows of length d; in = x fp32 [batch][ld_in] (length d).  For each
 *  token b and processed row n: out[b][n] = (accumulate ? out[b][n] : 0) +
 *  op value (see sffn_gemv_op) and, if key_out is set, key_out[b][n] =
 *  bits(out[b][n]) & 0x7FFFFFFF.  Entries of rows
 *  not processed are left untouched.  ld_out >= n_rows.  silu(z) = z / (1 +
 *  e^-z) as in the engine listing of [PowerInfer-2].  DOT_RELU uses W0 only
 *  (tau = tau_scale * ||x_b||_2, tau_scale >= 0); GATED uses W1 and aux fp32
 *  [batch][ld_aux] (aux_n read at processed rows only).  If rms_eps > 0 the
 *  row ops read each token through a unit-gain RMSNorm, x_b <- x_b /
 *  sqrt(mean(x_b^2) + rms_eps) (the pre-FFN normalisation of the Llama3 and
 *  Mixtral blocks the workloads are shaped like; fused, x is not modified);
 *  rms_eps = 0 uses x as given.  AXPY requires rms_eps = 0.
 *  DOT_RELU_CLUSTER ([PowerInfer-2] guide, "Neuron Cluster Decomposition":
 *  a cluster of `group` contiguous rows is active when any of its ReLU
 *  outputs is nonzero) processes every row (idx NULL, n_rows % group == 0)
 *  and raises key_out[n / group] (uint32 [n_rows / group], atomically) to
 *  the magnitude key of each nonzero out_n, so that with key_out zeroed
 *  beforehand it ends as the cluster's largest key (0 for an inactive
 *  cluster): the keys sparse_ffn_select ranks in cluster mode, without
 *  re-reading out (select's clear_keys re-zeroes them for the next call).
 *  GLU_RELU, PREDICT and DOT_RELU_CLUSTER run at batch 1 only.  PREDICT ([PowerInfer-2] guide,
 *  "Online Predictor": a linear classifier over the hidden state gives each
 *  neuron cluster an activation probability sigmoid(W_pred h + b), and the
 *  clusters above a threshold theta are the ones computed): W0 = W_pred
 *  [n_clusters][ld_w], aux = the bias fp32 [n_rows] (nullable: no bias),
 *  tau_scale = theta in (0, 1), no accumulate; out = the logits, and
 *  key_out[n] = 0 unless sigmoid(out_n) > theta holds for the fp32 logit in
 *  exact arithmetic, else the order-preserving key of out_n (nonzero), so a
 *  nonzero_only selection compacts the predicted clusters.
 *
 * AXPY: W0 is W_down^T, bf16 [n_rows][ld_w] with rows of length d (the
 *  output width); in = activations fp32 [batch][ld_in] (length n_rows);
 *  out[b][o] = (accumulate ? out[b][o] : 0) + alpha_b * sum over processed
 *  rows n of m_bn * in[b][n] * W0[n][o], with m_bn = row_mask[b][n] != 0 if
 *  row_mask (uint8 [batch][ld_mask]) is given, else 1, and alpha_b =
 *  alpha[b] (device fp32) if given, else 1.  ld_out >= d.  The row list is
 *  split over workgroups and the partial sums are added in a fixed order
 *  (a second kernel): results are bitwise reproducible run to run.
 *  Batch > 1 runs on MFMA (the gathered union as one dense block); the
 *  masked-out products contribute exactly zero.
 *
 * Limits: d % 8 == 0 (d % 32 == 0 when batch > 1), ld_w % 8 == 0, W0/W1/in/
 *  out 16-byte aligned, d <= 8192 for row ops at batch 1, 1 <= batch.
 *  With SFFN_PACKED in op: batch > 1 (EUNSUPPORTED otherwise), ld_w == d,
 *  d % 128 == 0 for row ops and d % 256 == 0 for AXPY (EUNSUPPORTED), and
 *  W0 / W1 hold sparse_ffn_packed_elems(n_rows, d, layout) elements.
 *  workspace: AXPY needs sparse_ffn_workspace_size(batch, rows, d) bytes
 *  (rows = k_max*group or n_rows).  Row ops at batch 1 take none (may be
 *  NULL).  Row ops at batch > 1 without an index list use it when given
 *  (256-byte aligned; sparse_ffn_workspace_size(batch, n_rows, d) bytes
 *  suffice): when the 32-row tile pairs do not split evenly over the CUs,
 *  the last pairs are split along K and a second kernel adds the slices in
 *  a fixed order (results stay reproducible run to run); without one, or
 *  if it is too small, the call runs unsplit.  It needs no initialisation.
 */
sffn_status sparse_ffn_gemv(int op,
                            const uint16_t* W0, const uint16_t* W1,
                            int n_rows, int d, int ld_w,
                            const float* in, int batch, int ld_in,
                            const int32_t* idx, const int32_t* count, int k_max, int group,
                            const uint8_t* row_mask, int ld_mask,
                            float tau_scale, float rms_eps,
                            const float* aux, int ld_aux,
                            const float* alpha,
                            float* out, uint32_t* key_out, int ld_out, int accumulate,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_ffn_gemv_keyed -- the batch-1 gathered product over the rows a
 * threshold selects ([SelectInfer] §5: only the selected neurons are read;
 * [LeanStream] "Permutation-Invariant Execution": the sum over neurons may
 * be taken in any grouping):
 *   out[o] = (accumulate ? out[o] : 0) + alpha * sum over n < n_rows with
 *            key_n > T or (key_n == T and n <= I) of in[n] * W[n][o],
 * where (T, I) = (thr[0], (int32) thr[1]) -- the output of
 * sparse_ffn_select_threshold -- and key_n is keys[n] read as key_type (the
 * keys that selection ranked).  W = W_down^T, bf16 [n_rows][ld_w] with rows
 * of length d; in fp32 [n_rows]; out fp32 [d].  Rows outside the selection
 * are never read.  The neurons are split over workgroups and waves by
 * index range; each wave forms its rows from the keys (no index list), and
 * the partial sums are added in a fixed order
 * (a second kernel): reproducible run to run, and the sum of
 * sparse_ffn_gemv over the selection's index list up to the order of fp32
 * additions.
 *  k_max     : an upper bound of the number of selected rows; it sizes the
 *              launch only (the threshold decides what is read).
 *  alpha     : nullable device fp32 scale.
 *  workspace : sparse_ffn_workspace_size(1, k_max, d) bytes, 256-byte
 *              aligned; needs no initialisation.
 * Limits: n_rows >= 1, d % 8 == 0, d >= 8, ld_w >= d, ld_w % 8 == 0,
 * 0 <= k_max <= n_rows; W / in / out 16-byte aligned, keys 4-byte, thr
 * 8-byte; n_rows up to 262,144 (EUNSUPPORTED above).
 */
sffn_status sparse_ffn_gemv_keyed(const uint16_t* W, int n_rows, int d, int ld_w,
                                  const float* in, const void* keys, int key_type,
                                  const uint32_t* thr, int k_max, const float* alpha,
                                  float* out, int accumulate,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_ffn_gemv_noalloc -- sparse_ffn_gemv without a workspace argument, for
 * callers that cannot allocate device memory: code recorded under HIP graph
 * capture, tight serving loops, and harnesses that forbid hipMalloc.  Same
 * arguments, operations, results and errors as sparse_ffn_gemv (it validates
 * and launches through it, so the results are bitwise those of
 * sparse_ffn_gemv); AXPY's split-K partials go to a static device array of
 * SFFN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it
 * runs on until the process ends.  The call allocates and frees nothing.
 *  - Limit: an AXPY whose sparse_ffn_workspace_size(batch, rows, d) exceeds
 *    SFFN_NOALLOC_SCRATCH_BYTES is rejected with SFFN_EWORKSPACE before any
 *    device work (e.g. batch 1 up to d of about 32K outputs; batch 16 at
 *    d = 5120).  Row ops need no scratch.
 *  - The array of the current device is used (its address is looked up once
 *    per device, with that device current); `stream` must belong to the
 *    current device.  The array needs no initialisation: every call writes
 *    the partials it reads.
 *  - All calls on one GPU share its array, which keeps the last call's
 *    contents: two calls that may run at the same time on one GPU (other
 *    streams, other host threads) race on it and give wrong results.
 *    Order such calls on one stream, or give them sparse_ffn_gemv with their
 *    own workspaces.
 */
#define SFFN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
sffn_status sparse_ffn_gemv_noalloc(int op,
                                    const uint16_t* W0, const uint16_t* W1,
                                    int n_rows, int d, int ld_w,
                                    const float* in, int batch, int ld_in,
                                    const int32_t* idx, const int32_t* count, int k_max, int group,
                                    const uint8_t* row_mask, int ld_mask,
                                    float tau_scale, float rms_eps,
                                    const float* aux, int ld_aux,
                                    const float* alpha,
                                    float* out, uint32_t* key_out, int ld_out, int accumulate,
                                    void* stream);

/*
 * sparse_ffn_fused_swiglu -- one sparse SwiGLU FFN at batch 1 in a single
 * pass per neuron ([SelectInfer] §5 computes only the neurons of the set U;
 * [LeanStream] "Permutation-Invariant Execution": the FFN output is a sum
 * over hidden neurons, so each neuron's contribution can be finished on its
 * own, in any order).  For every processed neuron n:
 *   a_n = silu(s * W_g[n].x) * (s * W_u[n].x),  silu(z) = z / (1 + e^-z),
 *   y   = (accumulate ? y : 0) + sum_n a_n * W_d[n],
 * with s = 1 / sqrt(mean(x^2) + rms_eps) if rms_eps > 0 (the unit-gain
 * RMSNorm of sparse_ffn_gemv's row ops), else s = 1.  Processed neurons:
 * all n < n_rows if idx is NULL (e.g. a set U compacted once per prompt
 * with sparse_ffn_compact, decoded with no indirection), otherwise idx[i]
 * for i < min(*count, k_max) (device int32, 0 <= idx[i] < n_rows, a
 * precondition the kernels do not check).  Skipped neurons are never read.
 *  Wg, Wu : bf16 [n_rows][ld_w], row n = neuron n's gate / up weights
 *           (length d).
 *  Wd     : bf16 [n_rows][ld_w], row n = W_down^T[n], the neuron's down
 *           weights over the d outputs (d_model in and out).  The three
 *           matrices share ld_w, so one record per neuron [gate | up | down]
 *           (ld_w = 3d, Wu = Wg + d, Wd = Wg + 2d) streams a layer as one
 *           sequential read.
 *  x      : fp32 [d]; y : fp32 [d]; x and y may be the same buffer (a
 *           residual stream updated in place): y is written by a second
 *           kernel after every read of x.
 *  a_out  : nullable fp32 [n_rows]: a_n at each processed neuron n; other
 *           entries are left untouched.
 *  workspace: sparse_ffn_workspace_size(1, rows, d) bytes, rows = k_max if
 *           idx is given, else n_rows; 256-byte aligned; no initialisation.
 *           The workgroups' partial sums are added in a fixed order (a
 *           second kernel): results are bitwise reproducible run to run.
 * Limits: d % 8 == 0, 8 <= d <= 4096 (EUNSUPPORTED above), ld_w >= d,
 * ld_w % 8 == 0, Wg / Wu / Wd / x / y 16-byte aligned, 0 <= k_max <=
 * n_rows.  Errors: EINVAL for a bad argument, EWORKSPACE for a missing or
 * short workspace; nothing is launched then.
 */
sffn_status sparse_ffn_fused_swiglu(const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                                    int n_rows, int d, int ld_w,
                                    const float* x, float rms_eps,
                                    const int32_t* idx, const int32_t* count, int k_max,
                                    float* a_out, float* y, int accumulate,
                                    void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_ffn_packed_elems -- bf16 elements of W [n_rows][d] in a packed
 * layout (sffn_layout); 0 if d does not fit the layout (ROW_TILES: d % 128
 * == 0; COL_PANELS: d % 256 == 0) or the layout is unknown.
 *
 * sparse_ffn_pack_weights -- out = W [n_rows][ld_w] (rows of length d)
 * re-laid in a packed layout, once per weight matrix (load time), for the
 * batched kernels' contiguous reads (sparse_ffn_gemv with SFFN_PACKED).  A
 * layout only orders the same weights differently: which rows a product
 * reads and what it computes are unchanged.
 *  W   : bf16, 16-byte aligned, ld_w >= d, ld_w % 8 == 0.
 *  out : bf16 [sparse_ffn_packed_elems(n_rows, d, layout)], 16-byte aligned,
 *        not overlapping W.
 * Errors: EINVAL for a bad argument or a layout d does not fit; nothing is
 * launched then.
 */
size_t sparse_ffn_packed_elems(int n_rows, int d, int layout);
sffn_status sparse_ffn_pack_weights(const uint16_t* W, int n_rows, int d, int ld_w, int layout,
                                    uint16_t* out, void* stream);

/*
 * sparse_ffn_row_norms -- out[r] = sqrt(sum_{o < d} W[r][o]^2) for each row r
 * of a bf16 matrix W [n_rows][ld_w] (rows of length d), accumulated in fp32
 * (offline).  For W^T of a projection (row j = input channel j) this is the
 * channel's weight norm ||W[:, j]||_2 that [WiSparse] multiplies with the
 * activation magnitude to rank channels (see key_scale of sparse_ffn_select).
 * Limits: d % 8 == 0, ld_w >= d, ld_w % 8 == 0, W 16-byte aligned.
 */
sffn_status sparse_ffn_row_norms(const uint16_t* W, int n_rows, int d, int ld_w, float* out,
                                 void* stream);

/*
 * sparse_ffn_gemv_lists -- one gathered product over several row lists into
 * one output, at batch 1.  The routed experts of a MoE layer add their FFN
 * outputs with the router's mixing weights ([PowerInfer-2] guide, the MoE
 * engine listing sums the selected experts' outputs); with every expert's
 * active rows as one list, their down products become one product:
 *   out[o] = (accumulate ? out[o] : 0)
 *            + sum_{l < n_lists} alpha_l * sum over processed rows n of list l
 *              of in_l[n] * W_l[n][o]
 * List l processes, for i < min(*count[l], k_max[l]) and g < group, row
 * idx[l][i]*group + g of W[l] (bf16 [n_rows[l]][ld_w], rows of length d,
 * 16-byte aligned); in[l] is fp32 [n_rows[l]]; alpha[l] is a device fp32
 * scalar, or NULL for 1.  W, n_rows, in, idx, count, k_max and alpha are
 * HOST arrays of n_lists entries (the pointers they hold are device
 * pointers; alpha itself may be NULL).  The lists share d, ld_w and group.
 * Rows of every list are split into chunks whose partial sums (scaled by
 * alpha_l) are added in a fixed order by a second kernel: bitwise
 * reproducible run to run.  Skipped rows are never read.
 * Limits: 1 <= n_lists <= 8; d % 8 == 0; ld_w >= d, ld_w % 8 == 0;
 * 0 <= k_max[l], k_max[l]*group <= n_rows[l]; out 16-byte aligned.
 * workspace: sparse_ffn_workspace_size(1, sum_l k_max[l]*group, d) bytes,
 * 256-byte aligned.  Errors as for sparse_ffn_gemv (nothing is launched on
 * a rejected call).
 */
sffn_status sparse_ffn_gemv_lists(int n_lists, const uint16_t* const* W, const int* n_rows,
                                  int d, int ld_w, const float* const* in,
                                  const int32_t* const* idx, const int32_t* const* count,
                                  const int* k_max, int group, const float* const* alpha,
                                  float* out, int accumulate,
                                  void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_ffn_rowop_lists -- one row op (GLU_SILU, DOT_RELU, GATED, DOT,
 * GLU_RELU or PREDICT, as in sparse_ffn_gemv) over several row lists at
 * batch 1, in one launch: the routed experts of a MoE layer are computed
 * on the same input ([PowerInfer-2] guide, MoE engine listing), so their
 * gates, ups or predictors can run as one pass instead of one call per
 * expert.  List l reads W0[l] / W1[l] (bf16 [n_rows][ld_w], rows of length
 * d, 16-byte aligned) at its rows -- all n_rows rows when idx is NULL, else
 * for i < min(*count[l], k_max[l]) and g < group, row idx[l][i]*group + g --
 * and writes out[l][row] (and key_out[l][row]) exactly as sparse_ffn_gemv
 * would for that list alone (bitwise the same values); aux[l] is GATED's
 * gate values or PREDICT's bias (fp32 [n_rows]).  x: fp32 [d], shared, read
 * through the optional RMSNorm (rms_eps).  W0, W1, idx, count, k_max, aux,
 * out and key_out are HOST arrays of n_lists entries holding device
 * pointers; W1 may be NULL unless the op uses it (GLU_SILU, GATED,
 * GLU_RELU), W0 may be NULL for GATED, idx NULL processes every row of
 * every list, aux NULL except for GATED, key_out NULL or with NULL entries.
 * tau_scale and accumulate as in sparse_ffn_gemv.
 * Limits: 1 <= n_lists <= 8; 8 <= d <= 5120, d % 8 == 0; ld_w >= d,
 * ld_w % 8 == 0; k_max[l]*group <= n_rows; x 16-byte aligned.  Errors as
 * for sparse_ffn_gemv (nothing is launched on a rejected call).
 */
sffn_status sparse_ffn_rowop_lists(int op, int n_lists, const uint16_t* const* W0,
                                   const uint16_t* const* W1, int n_rows, int d, int ld_w,
                                   const float* x, const int32_t* const* idx,
                                   const int32_t* const* count, const int* k_max, int group,
                                   float tau_scale, float rms_eps, const float* const* aux,
                                   float* const* out, uint32_t* const* key_out, int accumulate,
                                   void* stream);

/*
 * sparse_ffn_compact -- gather the weight rows of a selected neuron set into
 * a dense buffer, once per selection ([SelectInfer] §5 keeps the computed
 * set U fixed for a prompt's decode; [LeanStream] "Permutation-Invariant
 * Execution": a neuron subset is an ordinary dense matrix, in any order).
 *  W     : bf16 [n_rows][ld_w], rows of length d (d % 8 == 0, ld_w % 8 == 0).
 *  idx   : device int32 [k], rows to gather (0 <= idx[i] < n_rows), k from
 *          the host (k >= 0).
 *  transpose = 0: out bf16 [k][ld_out], out[i][0..d) = W[idx[i]][0..d)
 *          (ld_out >= d, % 8 == 0).
 *  transpose = 1: out bf16 [d][ld_out], out[o][i] = W[idx[i]][o] for i < k
 *          and 0 for k <= i < ld_out (ld_out >= k, % 8 == 0): the down
 *          weights of U output-major, for SFFN_OP_DOT.
 * W and out 16-byte aligned.
 */
sffn_status sparse_ffn_compact(const uint16_t* W, int n_rows, int d, int ld_w,
                               const int32_t* idx, int k, int transpose,
                               uint16_t* out, int ld_out, void* stream);

/*
 * sparse_ffn_gather -- dst[i] = src[idx[i]] for 4-byte elements (fp32,
 * uint32 or int32), i < min(*count, k_max) (k_max if count is NULL); the
 * rest of dst is untouched.  It carries per-neuron values into the
 * positions of a compacted subset: the index remap of a selectively loaded
 * layer ([SelectInfer] §4), whose resident weights keep only the loaded
 * neurons in ascending order, so that e.g. the base set can be ranked again
 * in the loaded positions, or positions mapped back to neuron ids.
 *  src   : device [n_src], n_src >= 1.
 *  idx   : device int32 [k_max]; an index outside [0, n_src) reads the
 *          nearest valid element (a precondition violation, not an error).
 *  count : nullable device int32 [1].
 *  dst   : device [k_max].  All 4-byte aligned; k_max >= 0.
 */
sffn_status sparse_ffn_gather(const void* src, int n_src, const int32_t* idx,
                              const int32_t* count, int k_max, void* dst, void* stream);

/*
 * Bytes of one middle-tier column record for d_out outputs in n_seg output
 * segments: a 16-byte header holding n_seg pairs (fp16 scale, fp16 zero),
 * then d_out/2 bytes of 4-bit codes (output 2i in the low nibble of byte i,
 * output 2i+1 in the high nibble), rounded up to 16 bytes.  n_seg <= 4.
 */
size_t sparse_ffn_tier_record_bytes(int d_out, int n_seg);

/*
 * sparse_ffn_encode_tiers -- the offline SpAx encoding (Fig 2, Fig 3): each
 * input column j (row j of W^T, bf16 [n_in][ld_w], length d_out) gets its
 * own 4-bit uniform codes, one (scale, zero) per output segment
 * [seg_rows[s], seg_rows[s+1]) (Q, K and V of Fig 4 are separate segments).
 *   zero  = fp16(min w);  scale = fp16(fp32(max w - zero) / 15);
 *   q     = clip(rint((w - zero) / scale), 0, 15) in fp32 (0 if scale == 0).
 * seg_rows is a HOST array [n_seg+1], 0 = seg_rows[0] < ... < seg_rows[n_seg]
 * = d_out, every boundary a multiple of 64.  mid_rec: uint8 [n_in][rec_bytes],
 * rec_bytes >= sparse_ffn_tier_record_bytes(d_out, n_seg), multiple of 16.
 */
sffn_status sparse_ffn_encode_tiers(const uint16_t* Wt, int ld_w, int n_in, int d_out,
                                    const int32_t* seg_rows, int n_seg,
                                    uint8_t* mid_rec, int rec_bytes, void* stream);

/*
 * sparse_ffn_tiered_gemv -- the SpAx three-tier read (abstract, Fig 2, Fig 3):
 *   y = (accumulate ? y : 0) + sum_{j in top} W^T[j][:] x_j
 *                             + sum_{j in mid} What^T[j][:] x_j,
 *   What^T[j][o] = zero_j,s + scale_j,s * q_j,o  (s = segment of output o);
 * columns in neither list are skipped and never read.  Wt bf16 [n_in][ld_w]
 * (rows of length d_out), mid_rec as written by sparse_ffn_encode_tiers,
 * x fp32 [n_in], y fp32 [d_out].  idx_top / idx_mid are the compacted
 * column lists of the two tiers (e.g. select ranges [0, k_top) and
 * [k_top, k_top + k_mid) of |x|), with device counts cnt_top / cnt_mid
 * (min(*cnt, k_max) entries used).  seg_rows is a HOST array as for the
 * encoder.  workspace: sparse_ffn_workspace_size(1, k_top_max + k_mid_max,
 * d_out) bytes.
 */
sffn_status sparse_ffn_tiered_gemv(const uint16_t* Wt, int ld_w,
                                   const uint8_t* mid_rec, int rec_bytes,
                                   const int32_t* seg_rows, int n_seg,
                                   int n_in, int d_out, const float* x,
                                   const int32_t* idx_top, const int32_t* cnt_top, int k_top_max,
                                   const int32_t* idx_mid, const int32_t* cnt_mid, int k_mid_max,
                                   float* y, int accumulate,
                                   void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_ffn_tiered_gemv_keyed -- sparse_ffn_tiered_gemv with the two tiers
 * given as threshold pairs (the output of sparse_ffn_select_threshold with
 * k_top and k) instead of column lists:
 *   top = { j : key_j > T_top, or key_j == T_top and j <= I_top },
 *   mid = { j : key_j > T, or key_j == T and j <= I } less top,
 * with (T_top, I_top) = thr_top[0..1], (T, I) = thr[0..1] (I read as int32)
 * and key_j = keys[j] read as key_type (the keys that selection ranked, e.g.
 * x itself with SFFN_KEY_ABS_F32).  y is that of sparse_ffn_tiered_gemv over
 * the two tiers' index lists up to the order of fp32 additions, and the same
 * bits run to run.  Each wave forms its columns from the keys; columns in
 * neither tier are never read.
 *  k_top_max, k_mid_max : upper bounds of the tier sizes; they size the
 *                         launch only.
 *  workspace            : sparse_ffn_workspace_size(1, k_top_max +
 *                         k_mid_max, d_out) bytes, 256-byte aligned.
 * Limits: those of sparse_ffn_tiered_gemv, n_in up to 524,288
 * (EUNSUPPORTED above); keys 4-byte aligned, thr_top / thr 8-byte aligned.
 */
sffn_status sparse_ffn_tiered_gemv_keyed(const uint16_t* Wt, int ld_w,
                                         const uint8_t* mid_rec, int rec_bytes,
                                         const int32_t* seg_rows, int n_seg,
                                         int n_in, int d_out, const float* x,
                                         const void* keys, int key_type,
                                         const uint32_t* thr_top, const uint32_t* thr,
                                         int k_top_max, int k_mid_max,
                                         float* y, int accumulate,
                                         void* workspace, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_FFN_H */
