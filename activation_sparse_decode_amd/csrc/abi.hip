// C ABI of libsparse_ffn.so: argument validation, error reporting and
// dispatch to the kernels.  Every check runs before anything is launched;
// a rejected call launches nothing.  See include/sparse_ffn.h for the
// contract of each entry point.
#include <cmath>
#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/sparse_ffn.h"
#include "sffn_splitk.h"

namespace {

thread_local std::string g_last_error;

sffn_status fail(sffn_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sffn_status ok() {
  g_last_error.clear();
  return SFFN_OK;
}

sffn_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SFFN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

// Device memory of the allocation-free gemv entry point: a file-scope array
// that each GPU holds (its own copy) from the library's load until the
// process ends.  In host code `scratch` only names the symbol; its device
// address on the current GPU comes from hipGetSymbolAddress, looked up once
// per device and kept in scratch_ptr[].
constexpr size_t kScratchBytes = SFFN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The scratch array's address on the current device (looked up on the first
// call per device, with that device current).
sffn_status current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SFFN_EHIP, "gemv_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SFFN_EUNSUPPORTED, "gemv_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SFFN_EHIP, "gemv_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return SFFN_OK;
}

// Checked mode (the environment variable SFFN_DEBUG_CHECKS set to anything
// but "0", read at every call): before a launch, a call that takes a device
// index list waits for its stream, reads the count and the list on the host
// and checks the preconditions the kernels rely on.  For debugging only: it
// synchronises and reads device memory, which the normal contract never does.
bool debug_checks() {
  const char* e = std::getenv("SFFN_DEBUG_CHECKS");
  return e && e[0] && !(e[0] == '0' && e[1] == '\0');
}

// The entries idx[i], i < min(*count, k_max) (k_max without a count), must be
// in [0, limit) and, if `distinct`, pairwise different; *count must be >= 0.
sffn_status check_list(const char* what, int list, const int32_t* idx, const int32_t* count,
                       int k_max, long limit, bool distinct, hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(SFFN_EHIP, "%s: debug check: %s", what, hipGetErrorString(e));
  int n = k_max;
  if (count) {
    int32_t c = 0;
    e = hipMemcpy(&c, count, sizeof(c), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(SFFN_EHIP, "%s: debug check: %s", what, hipGetErrorString(e));
    if (c < 0) return fail(SFFN_EINVAL, "%s: list %d: device count %d < 0 (debug check)", what, list, c);
    n = std::min(c, k_max);
  }
  if (n <= 0) return SFFN_OK;
  std::vector<int32_t> h((size_t)n);
  e = hipMemcpy(h.data(), idx, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SFFN_EHIP, "%s: debug check: %s", what, hipGetErrorString(e));
  std::vector<uint8_t> seen(distinct ? (size_t)std::max(limit, 0L) : 0);
  for (int i = 0; i < n; ++i) {
    if (h[i] < 0 || h[i] >= limit)
      return fail(SFFN_EINVAL, "%s: list %d: idx[%d] = %d outside [0, %ld) (debug check)", what,
                  list, i, h[i], limit);
    if (distinct) {
      if (seen[h[i]])
        return fail(SFFN_EINVAL, "%s: list %d: idx[%d] = %d repeats an earlier entry (debug check)",
                    what, list, i, h[i]);
      seen[h[i]] = 1;
    }
  }
  return SFFN_OK;
}

#define DEBUG_CHECK_LIST(...)                              \
  do {                                                     \
    if (debug_checks()) {                                  \
      const sffn_status st_ = check_list(__VA_ARGS__);     \
      if (st_ != SFFN_OK) return st_;                      \
    }                                                      \
  } while (0)

}  // namespace

namespace sffn {

size_t workspace_bytes(int batch, int n_rows, int d_out) {
  if (batch < 1) batch = 1;
  if (n_rows < 0) n_rows = 0;
  if (d_out < 0) d_out = 0;
  if (batch == 1) return kWsHeaderBytes + align256((size_t)kMaxSplit * d_out * sizeof(float));
  const int Mt = (batch + 15) / 16;
  const size_t Mpad = (size_t)Mt * 16;
  const size_t Kpad = ((size_t)n_rows + 63) / 64 * 64;
  return kWsHeaderBytes + align256((size_t)max_split_mfma(Mt) * Mpad * d_out * sizeof(float)) +
         2 * align256(Mpad * Kpad * 2);
}
}  // namespace sffn

extern "C" {

const char* sffn_last_error(void) { return g_last_error.c_str(); }

int sffn_abi_version(void) { return SFFN_ABI_VERSION; }

size_t sparse_ffn_workspace_size(int batch, int n_rows, int d_out) {
  return sffn::workspace_bytes(batch, n_rows, d_out);
}

size_t sparse_ffn_tier_record_bytes(int d_out, int n_seg) {
  if (d_out <= 0 || n_seg < 1 || n_seg > 4) return 0;
  const size_t b = 16 + (size_t)(d_out + 1) / 2;
  return (b + 15) / 16 * 16;
}

sffn_status sparse_ffn_score(int mode, const float* in, int T, int n, int ld, int cluster,
                             int accumulate, const int32_t* picked, int k, void* out,
                             void* stream) {
  REQUIRE(mode >= 0 && mode <= 2, SFFN_EINVAL, "score: unknown mode %d", mode);
  REQUIRE(in && out, SFFN_EINVAL, "score: in and out must be non-null");
  REQUIRE(T >= 0 && n >= 0, SFFN_EINVAL, "score: T=%d and n=%d must be >= 0", T, n);
  REQUIRE(ld >= n, SFFN_EINVAL, "score: ld=%d < n=%d", ld, n);
  REQUIRE(aligned(in, 4) && aligned(out, 4), SFFN_EINVAL, "score: in/out must be 4-byte aligned");
  if (mode == SFFN_SCORE_CLUSTER_MAX) {
    REQUIRE(cluster >= 1, SFFN_EINVAL, "score: cluster=%d must be >= 1", cluster);
    REQUIRE(n % cluster == 0, SFFN_EINVAL, "score: n=%d not a multiple of cluster=%d", n, cluster);
  }
  if (mode == SFFN_SCORE_SOFTMAX_PICKED) {
    REQUIRE(picked != nullptr, SFFN_EINVAL, "score: softmax needs the picked indices");
    REQUIRE(k >= 1 && k <= n, SFFN_EINVAL, "score: k=%d outside [1, n=%d]", k, n);
  }
  if (n == 0 || (T == 0 && mode != SFFN_SCORE_SUM_ABS)) return ok();
  return from_hip(sffn::launch_score(mode, in, T, n, ld, cluster, accumulate, picked, k, out,
                                     (hipStream_t)stream),
                  "score launch");
}

sffn_status sparse_ffn_select(const void* keys, int key_type, const float* key_scale, int rows,
                              int n, int ld,
                              int cluster, int r_lo, int r_hi, int nonzero_only,
                              const uint8_t* include_mask, const uint8_t* exclude_mask,
                              uint8_t* mask_out, int ld_mask,
                              int32_t* idx_out, int ld_idx, int32_t* count_out,
                              int32_t* idx_top_out, int ld_idx_top, int32_t* count_top_out,
                              uint32_t* freq_inout, int clear_keys, void* stream) {
  REQUIRE(keys != nullptr, SFFN_EINVAL, "select: keys must be non-null");
  REQUIRE(key_type >= 0 && key_type <= 2, SFFN_EINVAL, "select: unknown key type %d", key_type);
  REQUIRE(rows >= 0, SFFN_EINVAL, "select: rows=%d must be >= 0", rows);
  REQUIRE(n >= 1 && n <= 32768, SFFN_EUNSUPPORTED, "select: n=%d outside [1, 32768]", n);
  REQUIRE(cluster >= 1, SFFN_EINVAL, "select: cluster=%d must be >= 1", cluster);
  REQUIRE(cluster == 1 || n <= 4096, SFFN_EUNSUPPORTED,
          "select: n=%d clusters exceed 4096 (the cluster-mode limit)", n);
  REQUIRE(cluster == 1 || (long)n * cluster <= (1L << 30), SFFN_EUNSUPPORTED,
          "select: n*cluster=%ld values exceed 2^30 (the cluster-mode limit)", (long)n * cluster);
  REQUIRE((long)ld >= (long)n * cluster, SFFN_EINVAL, "select: ld=%d < n*cluster=%ld", ld,
          (long)n * cluster);
  REQUIRE(r_lo >= 0 && r_lo <= r_hi, SFFN_EINVAL, "select: need 0 <= r_lo=%d <= r_hi=%d", r_lo,
          r_hi);
  REQUIRE(!(nonzero_only && key_type == SFFN_KEY_F32), SFFN_EINVAL,
          "select: nonzero_only is not defined for signed keys");
  REQUIRE(aligned(keys, 4), SFFN_EINVAL, "select: keys must be 4-byte aligned");
  if (key_scale) {
    REQUIRE(key_type == SFFN_KEY_ABS_F32 && cluster == 1, SFFN_EINVAL,
            "select: key_scale needs SFFN_KEY_ABS_F32 keys and cluster == 1");
    REQUIRE(aligned(key_scale, 4), SFFN_EINVAL, "select: key_scale must be 4-byte aligned");
  }
  if (mask_out) REQUIRE(ld_mask >= n, SFFN_EINVAL, "select: ld_mask=%d < n=%d", ld_mask, n);
  if (idx_out) {
    const long need = include_mask ? (long)n : std::min((long)r_hi - r_lo, (long)n);
    REQUIRE(ld_idx >= need, SFFN_EINVAL, "select: ld_idx=%d < %ld", ld_idx, need);
    REQUIRE(aligned(idx_out, 4), SFFN_EINVAL, "select: idx_out must be 4-byte aligned");
  }
  if (idx_top_out) {
    const long need = std::min((long)r_lo, (long)n);
    REQUIRE(ld_idx_top >= need, SFFN_EINVAL, "select: ld_idx_top=%d < %ld", ld_idx_top, need);
    REQUIRE(aligned(idx_top_out, 4), SFFN_EINVAL, "select: idx_top_out must be 4-byte aligned");
  }
  if (count_out) REQUIRE(aligned(count_out, 4), SFFN_EINVAL, "select: count_out misaligned");
  if (count_top_out) REQUIRE(aligned(count_top_out, 4), SFFN_EINVAL, "select: count_top_out misaligned");
  if (freq_inout) REQUIRE(aligned(freq_inout, 4), SFFN_EINVAL, "select: freq misaligned");
  if (clear_keys)
    REQUIRE(cluster == 1 && !key_scale && (void*)freq_inout != keys, SFFN_EINVAL,
            "select: clear_keys needs cluster == 1, no key_scale and freq distinct from keys");
  if (rows == 0) return ok();
  sffn::SelectArgs a{keys, key_type, key_scale, rows, n, ld, cluster, r_lo, r_hi, nonzero_only ? 1 : 0,
                     include_mask, exclude_mask, mask_out, ld_mask, idx_out, ld_idx, count_out,
                     idx_top_out,
                     ld_idx_top, count_top_out, freq_inout, clear_keys ? 1 : 0};
  return from_hip(sffn::launch_select(a, (hipStream_t)stream), "select launch");
}

sffn_status sparse_ffn_select_threshold(const void* keys, int key_type, int rows, int n, int ld,
                                        int k_top, int k, uint32_t* thr_top_out, uint32_t* thr_out,
                                        void* stream) {
  REQUIRE(keys != nullptr, SFFN_EINVAL, "select_threshold: keys must be non-null");
  REQUIRE(key_type >= 0 && key_type <= 2, SFFN_EINVAL, "select_threshold: unknown key type %d",
          key_type);
  REQUIRE(rows >= 0, SFFN_EINVAL, "select_threshold: rows=%d must be >= 0", rows);
  REQUIRE(n >= 1 && n <= 32768, SFFN_EUNSUPPORTED, "select_threshold: n=%d outside [1, 32768]", n);
  REQUIRE(ld >= n, SFFN_EINVAL, "select_threshold: ld=%d < n=%d", ld, n);
  REQUIRE(k >= 0, SFFN_EINVAL, "select_threshold: k=%d must be >= 0", k);
  REQUIRE(k_top >= 0 && k_top <= k, SFFN_EINVAL, "select_threshold: k_top=%d outside [0, k=%d]",
          k_top, k);
  REQUIRE(aligned(keys, 4), SFFN_EINVAL, "select_threshold: keys must be 4-byte aligned");
  REQUIRE(thr_out != nullptr && aligned(thr_out, 8), SFFN_EINVAL,
          "select_threshold: thr_out must be non-null and 8-byte aligned");
  REQUIRE(thr_top_out == nullptr || aligned(thr_top_out, 8), SFFN_EINVAL,
          "select_threshold: thr_top_out must be 8-byte aligned");
  REQUIRE(k_top == 0 || thr_top_out != nullptr, SFFN_EINVAL,
          "select_threshold: k_top=%d > 0 needs thr_top_out", k_top);
  if (rows == 0) return ok();
  sffn::SelectArgs a{keys, key_type, nullptr, rows, n, ld, 1, k_top, k, 0,
                     nullptr, nullptr, nullptr, 0, nullptr, 0, nullptr,
                     nullptr, 0, nullptr, nullptr, 0, thr_out, thr_top_out};
  return from_hip(sffn::launch_select(a, (hipStream_t)stream), "select_threshold launch");
}

// sigmoid(z) > theta  <=>  z > ln(theta / (1 - theta)); with t the largest
// fp32 not above that logit, an fp32 z exceeds the exact logit exactly when
// z > t.
static float logit_threshold(float theta) {
  const double exact = std::log((double)theta / (1.0 - (double)theta));
  float t = (float)exact;
  if ((double)t > exact) t = std::nextafter(t, -INFINITY);
  return t;
}

sffn_status sparse_ffn_gemv(int op, const uint16_t* W0, const uint16_t* W1, int n_rows, int d,
                            int ld_w, const float* in, int batch, int ld_in, const int32_t* idx,
                            const int32_t* count, int k_max, int group, const uint8_t* row_mask,
                            int ld_mask, float tau_scale, float rms_eps, const float* aux, int ld_aux,
                            const float* alpha, float* out, uint32_t* key_out, int ld_out,
                            int accumulate, void* workspace, size_t ws_bytes, void* stream) {
  const int packed = (op & SFFN_PACKED) ? 1 : 0;
  const int mask_rows = (op & SFFN_MASKED_ROWS) ? 1 : 0;
  op &= ~(SFFN_PACKED | SFFN_MASKED_ROWS);
  REQUIRE(op >= 0 && op <= 7, SFFN_EINVAL, "gemv: unknown op %d", op);
  REQUIRE(in && out, SFFN_EINVAL, "gemv: in and out must be non-null");
  REQUIRE(n_rows >= 0, SFFN_EINVAL, "gemv: n_rows=%d must be >= 0", n_rows);
  REQUIRE(d >= 8 && d % 8 == 0, SFFN_EINVAL, "gemv: d=%d must be a positive multiple of 8", d);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL, "gemv: ld_w=%d must be >= d and a multiple of 8",
          ld_w);
  REQUIRE(batch >= 1, SFFN_EINVAL, "gemv: batch=%d must be >= 1", batch);
  REQUIRE(batch == 1 || d % 32 == 0, SFFN_EUNSUPPORTED, "gemv: batch > 1 needs d %% 32 == 0 (d=%d)",
          d);
  REQUIRE(aligned(in, 16) && aligned(out, 16), SFFN_EINVAL, "gemv: in/out must be 16-byte aligned");
  if (batch > 1) REQUIRE(ld_in % 4 == 0, SFFN_EINVAL, "gemv: ld_in=%d must be a multiple of 4", ld_in);
  if (idx) {
    REQUIRE(count != nullptr, SFFN_EINVAL, "gemv: idx needs a device count");
    REQUIRE(group >= 1, SFFN_EINVAL, "gemv: group=%d must be >= 1", group);
    REQUIRE(k_max >= 0 && (long)k_max * group <= n_rows, SFFN_EINVAL,
            "gemv: k_max=%d * group=%d exceeds n_rows=%d", k_max, group, n_rows);
    REQUIRE(aligned(idx, 4) && aligned(count, 4), SFFN_EINVAL, "gemv: idx/count misaligned");
  }
  if (packed) {
    REQUIRE(batch > 1, SFFN_EUNSUPPORTED,
            "gemv: packed weights are read by the batched kernels only (batch > 1)");
    REQUIRE(ld_w == d, SFFN_EINVAL, "gemv: packed weights take ld_w == d (d=%d, ld_w=%d)", d, ld_w);
    if (op == SFFN_OP_AXPY)
      REQUIRE(d % 256 == 0, SFFN_EUNSUPPORTED, "gemv: packed AXPY weights need d %% 256 == 0 (d=%d)",
              d);
    else
      REQUIRE(d % 128 == 0, SFFN_EUNSUPPORTED,
              "gemv: packed row-op weights need d %% 128 == 0 (d=%d)", d);
  }
  if (mask_rows) {
    REQUIRE(op == SFFN_OP_AXPY, SFFN_EINVAL, "gemv: SFFN_MASKED_ROWS applies to AXPY only");
    REQUIRE(batch > 1, SFFN_EUNSUPPORTED, "gemv: SFFN_MASKED_ROWS needs batch > 1");
    REQUIRE(!idx, SFFN_EINVAL, "gemv: SFFN_MASKED_ROWS takes no index list (idx must be NULL)");
    REQUIRE(row_mask != nullptr, SFFN_EINVAL, "gemv: SFFN_MASKED_ROWS needs row_mask");
    REQUIRE(aligned(row_mask, 16) && ld_mask % 16 == 0, SFFN_EINVAL,
            "gemv: SFFN_MASKED_ROWS needs row_mask 16-byte aligned and ld_mask %% 16 == 0 "
            "(ld_mask=%d)", ld_mask);
  }
  const long items = idx ? (long)k_max * group : (long)n_rows;
  hipStream_t s = (hipStream_t)stream;

  if (op != SFFN_OP_AXPY) {
    if (op != SFFN_OP_GATED)
      REQUIRE(W0 && aligned(W0, 16), SFFN_EINVAL, "gemv: W0 must be non-null and 16-byte aligned");
    if (op == SFFN_OP_GLU_SILU || op == SFFN_OP_GATED || op == SFFN_OP_GLU_RELU)
      REQUIRE(W1 && aligned(W1, 16), SFFN_EINVAL, "gemv: W1 must be non-null and 16-byte aligned");
    if (op == SFFN_OP_GLU_RELU || op == SFFN_OP_PREDICT || op == SFFN_OP_DOT_RELU_CLUSTER)
      REQUIRE(batch == 1, SFFN_EUNSUPPORTED, "gemv: op %d runs at batch 1 only", op);
    if (op == SFFN_OP_DOT_RELU_CLUSTER) {
      REQUIRE(!idx, SFFN_EUNSUPPORTED, "gemv: DOT_RELU_CLUSTER processes every row (idx must be NULL)");
      REQUIRE(group >= 1 && n_rows % group == 0, SFFN_EINVAL,
              "gemv: DOT_RELU_CLUSTER needs group >= 1 dividing n_rows=%d (group=%d)", n_rows, group);
    }
    REQUIRE(ld_in >= d, SFFN_EINVAL, "gemv: ld_in=%d < d=%d", ld_in, d);
    REQUIRE(ld_out >= n_rows, SFFN_EINVAL, "gemv: ld_out=%d < n_rows=%d", ld_out, n_rows);
    REQUIRE(batch > 1 || d <= 8192, SFFN_EUNSUPPORTED, "gemv: d=%d > 8192 at batch 1", d);
    REQUIRE(rms_eps >= 0.f && std::isfinite(rms_eps), SFFN_EINVAL,
            "gemv: rms_eps must be finite and >= 0");
    if (op == SFFN_OP_DOT_RELU || op == SFFN_OP_GLU_RELU || op == SFFN_OP_DOT_RELU_CLUSTER)
      REQUIRE(tau_scale >= 0.f && std::isfinite(tau_scale), SFFN_EINVAL,
              "gemv: tau_scale must be finite and >= 0");
    if (op == SFFN_OP_PREDICT) {
      REQUIRE(tau_scale > 0.f && tau_scale < 1.f, SFFN_EINVAL,
              "gemv: PREDICT takes a probability threshold in (0, 1) as tau_scale");
      REQUIRE(!accumulate, SFFN_EINVAL, "gemv: PREDICT does not accumulate");
      if (aux) REQUIRE(ld_aux >= n_rows && aligned(aux, 4), SFFN_EINVAL,
                       "gemv: PREDICT bias needs ld_aux >= n_rows and 4-byte alignment");
      tau_scale = logit_threshold(tau_scale);
    }
    if (op == SFFN_OP_GATED) {
      REQUIRE(aux != nullptr, SFFN_EINVAL, "gemv: GATED needs aux");
      REQUIRE(ld_aux >= n_rows, SFFN_EINVAL, "gemv: ld_aux=%d < n_rows=%d", ld_aux, n_rows);
    }
    if (key_out) REQUIRE(aligned(key_out, 4), SFFN_EINVAL, "gemv: key_out misaligned");
    if (items == 0) return ok();
    if (batch > 1 && workspace)
      REQUIRE(aligned(workspace, 256), SFFN_EINVAL, "gemv: workspace must be 256-byte aligned");
    if (idx) DEBUG_CHECK_LIST("gemv", 0, idx, count, k_max, (long)n_rows / group, true, s);
    sffn::RowOpArgs a{op, W0, W1, n_rows, d, ld_w, in, batch, ld_in, idx, count, k_max,
                      (idx || op == SFFN_OP_DOT_RELU_CLUSTER) ? group : 1, tau_scale, rms_eps,
                      aux, ld_aux, out, key_out,
                      ld_out, accumulate ? 1 : 0, batch > 1 ? workspace : nullptr,
                      batch > 1 && workspace ? ws_bytes : 0, packed};
    return from_hip(batch == 1 ? sffn::launch_rowop_b1(a, s) : sffn::launch_rowop_mfma(a, s),
                    "gemv launch");
  }

  REQUIRE(W0 && aligned(W0, 16), SFFN_EINVAL, "gemv: W0 must be non-null and 16-byte aligned");
  REQUIRE(rms_eps == 0.f, SFFN_EINVAL, "gemv: AXPY takes no input normalisation (rms_eps must be 0)");
  REQUIRE(ld_in >= n_rows, SFFN_EINVAL, "gemv: ld_in=%d < n_rows=%d", ld_in, n_rows);
  REQUIRE(ld_out >= d, SFFN_EINVAL, "gemv: ld_out=%d < d=%d", ld_out, d);
  if (row_mask) REQUIRE(ld_mask >= n_rows, SFFN_EINVAL, "gemv: ld_mask=%d < n_rows=%d", ld_mask,
                        n_rows);
  if (alpha) REQUIRE(aligned(alpha, 4), SFFN_EINVAL, "gemv: alpha misaligned");
  const size_t need = sffn::workspace_bytes(batch, (int)items, d);
  REQUIRE(workspace != nullptr && ws_bytes >= need, SFFN_EWORKSPACE,
          "gemv: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  REQUIRE(aligned(workspace, 256), SFFN_EINVAL, "gemv: workspace must be 256-byte aligned");
  if (idx) DEBUG_CHECK_LIST("gemv", 0, idx, count, k_max, (long)n_rows / group, true, s);
  sffn::AxpyArgs a{W0, n_rows, d, ld_w, in, batch, ld_in, idx, count, k_max, idx ? group : 1,
                   row_mask, ld_mask, alpha, out, ld_out, accumulate ? 1 : 0, workspace, ws_bytes,
                   packed, mask_rows};
  return from_hip(batch == 1 ? sffn::launch_axpy_b1(a, s) : sffn::launch_axpy_mfma(a, s),
                  "gemv launch");
}

sffn_status sparse_ffn_fused_swiglu(const uint16_t* Wg, const uint16_t* Wu, const uint16_t* Wd,
                                    int n_rows, int d, int ld_w, const float* x, float rms_eps,
                                    const int32_t* idx, const int32_t* count, int k_max,
                                    float* a_out, float* y, int accumulate, void* workspace,
                                    size_t ws_bytes, void* stream) {
  REQUIRE(Wg && Wu && Wd, SFFN_EINVAL, "fused_swiglu: Wg, Wu and Wd must be non-null");
  REQUIRE(aligned(Wg, 16) && aligned(Wu, 16) && aligned(Wd, 16), SFFN_EINVAL,
          "fused_swiglu: Wg/Wu/Wd must be 16-byte aligned");
  REQUIRE(x && y, SFFN_EINVAL, "fused_swiglu: x and y must be non-null");
  REQUIRE(aligned(x, 16) && aligned(y, 16), SFFN_EINVAL, "fused_swiglu: x/y must be 16-byte aligned");
  REQUIRE(n_rows >= 0, SFFN_EINVAL, "fused_swiglu: n_rows=%d must be >= 0", n_rows);
  REQUIRE(d >= 8 && d % 8 == 0, SFFN_EINVAL, "fused_swiglu: d=%d must be a positive multiple of 8", d);
  REQUIRE(d <= 4096, SFFN_EUNSUPPORTED, "fused_swiglu: d=%d > 4096", d);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL,
          "fused_swiglu: ld_w=%d must be >= d and a multiple of 8", ld_w);
  REQUIRE(rms_eps >= 0.f && std::isfinite(rms_eps), SFFN_EINVAL,
          "fused_swiglu: rms_eps must be finite and >= 0");
  if (idx) {
    REQUIRE(count != nullptr, SFFN_EINVAL, "fused_swiglu: idx needs a device count");
    REQUIRE(k_max >= 0 && k_max <= n_rows, SFFN_EINVAL, "fused_swiglu: k_max=%d outside [0, n_rows=%d]",
            k_max, n_rows);
    REQUIRE(aligned(idx, 4) && aligned(count, 4), SFFN_EINVAL, "fused_swiglu: idx/count misaligned");
  }
  if (a_out) REQUIRE(aligned(a_out, 4), SFFN_EINVAL, "fused_swiglu: a_out misaligned");
  const long items = idx ? (long)k_max : (long)n_rows;
  const size_t need = sffn::workspace_bytes(1, (int)items, d);
  REQUIRE(workspace != nullptr && ws_bytes >= need, SFFN_EWORKSPACE,
          "fused_swiglu: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  REQUIRE(aligned(workspace, 256), SFFN_EINVAL, "fused_swiglu: workspace must be 256-byte aligned");
  if (idx)
    DEBUG_CHECK_LIST("fused_swiglu", 0, idx, count, k_max, n_rows, true, (hipStream_t)stream);
  sffn::FusedArgs a{Wg, Wu, Wd, ld_w, n_rows, d, x, rms_eps, idx, count, k_max, a_out, y,
                    accumulate ? 1 : 0, workspace, ws_bytes};
  return from_hip(sffn::launch_fused_swiglu(a, (hipStream_t)stream), "fused_swiglu launch");
}

size_t sparse_ffn_packed_elems(int n_rows, int d, int layout) {
  return sffn::packed_elems(n_rows, d, layout);
}

sffn_status sparse_ffn_pack_weights(const uint16_t* W, int n_rows, int d, int ld_w, int layout,
                                    uint16_t* out, void* stream) {
  REQUIRE(W && out, SFFN_EINVAL, "pack: W and out must be non-null");
  REQUIRE(layout == SFFN_LAYOUT_ROW_TILES || layout == SFFN_LAYOUT_COL_PANELS, SFFN_EINVAL,
          "pack: unknown layout %d", layout);
  REQUIRE(n_rows >= 0, SFFN_EINVAL, "pack: n_rows=%d must be >= 0", n_rows);
  REQUIRE(d > 0 && d % (layout == SFFN_LAYOUT_ROW_TILES ? 128 : 256) == 0, SFFN_EINVAL,
          "pack: d=%d must be a positive multiple of %d for layout %d", d,
          layout == SFFN_LAYOUT_ROW_TILES ? 128 : 256, layout);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL, "pack: ld_w=%d must be >= d and a multiple of 8",
          ld_w);
  REQUIRE(aligned(W, 16) && aligned(out, 16), SFFN_EINVAL, "pack: W/out must be 16-byte aligned");
  const size_t n_out = sffn::packed_elems(n_rows, d, layout);
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(W), o0 = reinterpret_cast<uintptr_t>(out);
  const uintptr_t w1 = w0 + 2 * ((n_rows > 0 ? (size_t)(n_rows - 1) * ld_w : 0) + (size_t)d);
  REQUIRE(o0 + 2 * n_out <= w0 || o0 >= w1, SFFN_EINVAL, "pack: out overlaps W");
  return from_hip(sffn::launch_pack(W, n_rows, d, ld_w, layout, out, (hipStream_t)stream),
                  "pack launch");
}

sffn_status sparse_ffn_row_norms(const uint16_t* W, int n_rows, int d, int ld_w, float* out,
                                 void* stream) {
  REQUIRE(W && out, SFFN_EINVAL, "row_norms: W and out must be non-null");
  REQUIRE(n_rows >= 0, SFFN_EINVAL, "row_norms: n_rows=%d must be >= 0", n_rows);
  REQUIRE(d >= 8 && d % 8 == 0, SFFN_EINVAL, "row_norms: d=%d must be a positive multiple of 8", d);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL,
          "row_norms: ld_w=%d must be >= d and a multiple of 8", ld_w);
  REQUIRE(aligned(W, 16) && aligned(out, 4), SFFN_EINVAL, "row_norms: W/out misaligned");
  if (n_rows == 0) return ok();
  return from_hip(sffn::launch_row_norms(W, n_rows, d, ld_w, out, (hipStream_t)stream),
                  "row_norms launch");
}

sffn_status sparse_ffn_rowop_lists(int op, int n_lists, const uint16_t* const* W0,
                                  const uint16_t* const* W1, int n_rows, int d, int ld_w,
                                  const float* x, const int32_t* const* idx,
                                  const int32_t* const* count, const int* k_max, int group,
                                  float tau_scale, float rms_eps, const float* const* aux,
                                  float* const* out, uint32_t* const* key_out, int accumulate,
                                  void* stream) {
  REQUIRE(op >= 0 && op <= 7 && op != SFFN_OP_AXPY, SFFN_EINVAL,
          "rowop_lists: op %d is not a row op", op);
  if (op == SFFN_OP_DOT_RELU_CLUSTER) {
    REQUIRE(!idx, SFFN_EUNSUPPORTED, "rowop_lists: DOT_RELU_CLUSTER processes every row (idx NULL)");
    REQUIRE(group >= 1 && n_rows % group == 0, SFFN_EINVAL,
            "rowop_lists: DOT_RELU_CLUSTER needs group >= 1 dividing n_rows=%d (group=%d)", n_rows,
            group);
  }
  REQUIRE(n_lists >= 1 && n_lists <= sffn::kMaxRowLists, SFFN_EINVAL,
          "rowop_lists: n_lists=%d must be in [1, %d]", n_lists, sffn::kMaxRowLists);
  REQUIRE(out != nullptr, SFFN_EINVAL, "rowop_lists: out (host array) must be non-null");
  REQUIRE(x && aligned(x, 16), SFFN_EINVAL, "rowop_lists: x must be non-null, 16-byte aligned");
  REQUIRE(n_rows >= 0, SFFN_EINVAL, "rowop_lists: n_rows=%d must be >= 0", n_rows);
  REQUIRE(d >= 8 && d % 8 == 0, SFFN_EINVAL, "rowop_lists: d=%d must be a positive multiple of 8", d);
  REQUIRE(d <= 5120, SFFN_EUNSUPPORTED, "rowop_lists: d=%d > 5120", d);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL,
          "rowop_lists: ld_w=%d must be >= d and a multiple of 8", ld_w);
  REQUIRE(rms_eps >= 0.f && std::isfinite(rms_eps), SFFN_EINVAL,
          "rowop_lists: rms_eps must be finite and >= 0");
  const bool use0 = op != SFFN_OP_GATED;
  const bool use1 = op == SFFN_OP_GLU_SILU || op == SFFN_OP_GATED || op == SFFN_OP_GLU_RELU;
  REQUIRE(!use0 || W0, SFFN_EINVAL, "rowop_lists: W0 (host array) must be non-null");
  REQUIRE(!use1 || W1, SFFN_EINVAL, "rowop_lists: W1 (host array) must be non-null");
  REQUIRE(op != SFFN_OP_GATED || aux, SFFN_EINVAL, "rowop_lists: GATED needs aux");
  if (idx) {
    REQUIRE(count && k_max, SFFN_EINVAL, "rowop_lists: idx needs count and k_max (host arrays)");
    REQUIRE(group >= 1, SFFN_EINVAL, "rowop_lists: group=%d must be >= 1", group);
  }
  if (op == SFFN_OP_DOT_RELU || op == SFFN_OP_GLU_RELU || op == SFFN_OP_DOT_RELU_CLUSTER)
    REQUIRE(tau_scale >= 0.f && std::isfinite(tau_scale), SFFN_EINVAL,
            "rowop_lists: tau_scale must be finite and >= 0");
  if (op == SFFN_OP_PREDICT) {
    REQUIRE(tau_scale > 0.f && tau_scale < 1.f, SFFN_EINVAL,
            "rowop_lists: PREDICT takes a probability threshold in (0, 1) as tau_scale");
    REQUIRE(!accumulate, SFFN_EINVAL, "rowop_lists: PREDICT does not accumulate");
    tau_scale = logit_threshold(tau_scale);
  }
  sffn::RowOpListsArgs L{};
  L.base = sffn::RowOpArgs{op, nullptr, nullptr, n_rows, d, ld_w, x, 1, d, nullptr, nullptr, 0,
                           (idx || op == SFFN_OP_DOT_RELU_CLUSTER) ? group : 1, tau_scale,
                           rms_eps, nullptr, n_rows, nullptr, nullptr,
                           n_rows, accumulate ? 1 : 0};
  L.n = n_lists;
  long items = 0;
  for (int l = 0; l < n_lists; ++l) {
    if (use0) REQUIRE(W0[l] && aligned(W0[l], 16), SFFN_EINVAL,
                      "rowop_lists: W0[%d] must be non-null and 16-byte aligned", l);
    if (use1) REQUIRE(W1[l] && aligned(W1[l], 16), SFFN_EINVAL,
                      "rowop_lists: W1[%d] must be non-null and 16-byte aligned", l);
    REQUIRE(out[l] && aligned(out[l], 4), SFFN_EINVAL, "rowop_lists: out[%d] must be non-null", l);
    if (key_out) REQUIRE(aligned(key_out[l], 4), SFFN_EINVAL, "rowop_lists: key_out[%d] misaligned", l);
    if (aux) REQUIRE(aligned(aux[l], 4), SFFN_EINVAL, "rowop_lists: aux[%d] misaligned", l);
    if (op == SFFN_OP_GATED) REQUIRE(aux[l] != nullptr, SFFN_EINVAL, "rowop_lists: aux[%d] is null", l);
    if (idx) {
      REQUIRE(idx[l] && count[l] && aligned(idx[l], 4) && aligned(count[l], 4), SFFN_EINVAL,
              "rowop_lists: idx[%d] / count[%d] must be non-null and 4-byte aligned", l, l);
      REQUIRE(k_max[l] >= 0 && (long)k_max[l] * group <= n_rows, SFFN_EINVAL,
              "rowop_lists: k_max[%d]=%d * group=%d exceeds n_rows=%d", l, k_max[l], group, n_rows);
      items += (long)k_max[l] * group;
    } else {
      items += n_rows;
    }
    L.W0[l] = use0 ? W0[l] : nullptr;
    L.W1[l] = use1 ? W1[l] : (use0 ? W0[l] : nullptr);
    L.idx[l] = idx ? idx[l] : nullptr;
    L.count[l] = idx ? count[l] : nullptr;
    L.k_max[l] = idx ? k_max[l] : 0;
    L.aux[l] = aux ? aux[l] : nullptr;
    L.out[l] = out[l];
    L.key_out[l] = key_out ? key_out[l] : nullptr;
  }
  if (!use0)
    for (int l = 0; l < n_lists; ++l) L.W0[l] = W1[l];   // GATED reads W1 only
  if (items == 0) return ok();
  if (idx)
    for (int l = 0; l < n_lists; ++l)
      DEBUG_CHECK_LIST("rowop_lists", l, idx[l], count[l], k_max[l], (long)n_rows / group, true,
                       (hipStream_t)stream);
  return from_hip(sffn::launch_rowop_lists(L, (hipStream_t)stream), "rowop_lists launch");
}

sffn_status sparse_ffn_gemv_lists(int n_lists, const uint16_t* const* W, const int* n_rows,
                                  int d, int ld_w, const float* const* in,
                                  const int32_t* const* idx, const int32_t* const* count,
                                  const int* k_max, int group, const float* const* alpha,
                                  float* out, int accumulate, void* workspace, size_t ws_bytes,
                                  void* stream) {
  REQUIRE(n_lists >= 1 && n_lists <= sffn::kMaxLists, SFFN_EINVAL,
          "gemv_lists: n_lists=%d must be in [1, %d]", n_lists, sffn::kMaxLists);
  REQUIRE(W && n_rows && in && idx && count && k_max, SFFN_EINVAL,
          "gemv_lists: W, n_rows, in, idx, count and k_max (host arrays) must be non-null");
  REQUIRE(out && aligned(out, 16), SFFN_EINVAL, "gemv_lists: out must be non-null, 16-byte aligned");
  REQUIRE(d >= 8 && d % 8 == 0, SFFN_EINVAL, "gemv_lists: d=%d must be a positive multiple of 8", d);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL,
          "gemv_lists: ld_w=%d must be >= d and a multiple of 8", ld_w);
  REQUIRE(group >= 1, SFFN_EINVAL, "gemv_lists: group=%d must be >= 1", group);
  sffn::AxpyListsArgs a{};
  long items = 0;
  for (int l = 0; l < n_lists; ++l) {
    REQUIRE(W[l] && aligned(W[l], 16), SFFN_EINVAL,
            "gemv_lists: W[%d] must be non-null and 16-byte aligned", l);
    REQUIRE(in[l] && aligned(in[l], 4), SFFN_EINVAL, "gemv_lists: in[%d] must be non-null", l);
    REQUIRE(idx[l] && count[l] && aligned(idx[l], 4) && aligned(count[l], 4), SFFN_EINVAL,
            "gemv_lists: idx[%d] and count[%d] must be non-null and 4-byte aligned", l, l);
    REQUIRE(n_rows[l] >= 0 && k_max[l] >= 0 && (long)k_max[l] * group <= n_rows[l], SFFN_EINVAL,
            "gemv_lists: list %d: k_max=%d * group=%d exceeds n_rows=%d", l, k_max[l], group,
            n_rows[l]);
    const float* al = alpha ? alpha[l] : nullptr;
    if (al) REQUIRE(aligned(al, 4), SFFN_EINVAL, "gemv_lists: alpha[%d] misaligned", l);
    a.l[l] = sffn::AxpyList{W[l], in[l], idx[l], count[l], al, k_max[l]};
    items += (long)k_max[l] * group;
  }
  REQUIRE(items <= INT32_MAX, SFFN_EINVAL, "gemv_lists: too many rows");
  const size_t need = sffn::workspace_bytes(1, (int)items, d);
  REQUIRE(workspace != nullptr && ws_bytes >= need, SFFN_EWORKSPACE,
          "gemv_lists: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  REQUIRE(aligned(workspace, 256), SFFN_EINVAL, "gemv_lists: workspace must be 256-byte aligned");
  a.n = n_lists;
  a.d = d;
  a.ld_w = ld_w;
  a.group = group;
  a.out = out;
  a.accumulate = accumulate ? 1 : 0;
  a.ws = workspace;
  a.ws_bytes = ws_bytes;
  for (int l = 0; l < n_lists; ++l)
    DEBUG_CHECK_LIST("gemv_lists", l, idx[l], count[l], k_max[l], (long)n_rows[l] / group, true,
                     (hipStream_t)stream);
  return from_hip(sffn::launch_axpy_lists(a, (hipStream_t)stream), "gemv_lists launch");
}

sffn_status sparse_ffn_gather(const void* src, int n_src, const int32_t* idx, const int32_t* count,
                              int k_max, void* dst, void* stream) {
  REQUIRE(n_src >= 1, SFFN_EINVAL, "gather: n_src=%d must be >= 1", n_src);
  REQUIRE(k_max >= 0, SFFN_EINVAL, "gather: k_max=%d must be >= 0", k_max);
  REQUIRE(src && dst && (k_max == 0 || idx), SFFN_EINVAL, "gather: src, dst and idx must be non-null");
  REQUIRE(aligned(src, 4) && aligned(dst, 4) && aligned(idx, 4) && aligned(count, 4), SFFN_EINVAL,
          "gather: src/dst/idx/count must be 4-byte aligned");
  if (k_max == 0) return ok();
  return from_hip(sffn::launch_gather32(static_cast<const uint32_t*>(src), n_src, idx, count, k_max,
                                        static_cast<uint32_t*>(dst), (hipStream_t)stream),
                  "gather launch");
}

sffn_status sparse_ffn_compact(const uint16_t* W, int n_rows, int d, int ld_w,
                               const int32_t* idx, int k, int transpose, uint16_t* out,
                               int ld_out, void* stream) {
  REQUIRE(W && out, SFFN_EINVAL, "compact: W and out must be non-null");
  REQUIRE(n_rows >= 0 && k >= 0 && k <= n_rows, SFFN_EINVAL,
          "compact: need 0 <= k=%d <= n_rows=%d", k, n_rows);
  REQUIRE(k == 0 || idx != nullptr, SFFN_EINVAL, "compact: idx must be non-null");
  REQUIRE(d >= 8 && d % 8 == 0, SFFN_EINVAL, "compact: d=%d must be a positive multiple of 8", d);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL, "compact: ld_w=%d must be >= d, %% 8", ld_w);
  REQUIRE(ld_out % 8 == 0 && ld_out >= (transpose ? k : d), SFFN_EINVAL,
          "compact: ld_out=%d must be a multiple of 8 and >= %d", ld_out, transpose ? k : d);
  REQUIRE(aligned(W, 16) && aligned(out, 16), SFFN_EINVAL, "compact: W/out must be 16-byte aligned");
  if (idx) REQUIRE(aligned(idx, 4), SFFN_EINVAL, "compact: idx misaligned");
  if (transpose && ld_out == 0) return ok();
  if (k > 0) DEBUG_CHECK_LIST("compact", 0, idx, nullptr, k, n_rows, false, (hipStream_t)stream);
  return from_hip(sffn::launch_compact(W, ld_w, d, idx, k, transpose ? 1 : 0, out, ld_out,
                                       (hipStream_t)stream),
                  "compact launch");
}

static sffn_status check_segments(const char* who, const int32_t* seg_rows, int n_seg, int d_out) {
  REQUIRE(seg_rows != nullptr, SFFN_EINVAL, "%s: seg_rows (host) must be non-null", who);
  REQUIRE(n_seg >= 1 && n_seg <= 4, SFFN_EUNSUPPORTED, "%s: n_seg=%d outside [1, 4]", who, n_seg);
  REQUIRE(seg_rows[0] == 0 && seg_rows[n_seg] == d_out, SFFN_EINVAL,
          "%s: segments must start at 0 and end at d_out=%d", who, d_out);
  for (int i = 0; i < n_seg; ++i) {
    REQUIRE(seg_rows[i + 1] > seg_rows[i], SFFN_EINVAL, "%s: segments must increase", who);
    REQUIRE(seg_rows[i + 1] % 64 == 0, SFFN_EINVAL, "%s: segment bound %d not a multiple of 64", who,
            seg_rows[i + 1]);
  }
  return ok();
}

sffn_status sparse_ffn_encode_tiers(const uint16_t* Wt, int ld_w, int n_in, int d_out,
                                    const int32_t* seg_rows, int n_seg, uint8_t* mid_rec,
                                    int rec_bytes, void* stream) {
  REQUIRE(Wt && mid_rec, SFFN_EINVAL, "encode: Wt and mid_rec must be non-null");
  REQUIRE(n_in >= 0 && d_out >= 64 && d_out % 64 == 0, SFFN_EINVAL,
          "encode: need n_in >= 0 and d_out a positive multiple of 64 (d_out=%d)", d_out);
  REQUIRE(ld_w >= d_out && ld_w % 8 == 0, SFFN_EINVAL, "encode: ld_w=%d must be >= d_out, %% 8",
          ld_w);
  sffn_status st = check_segments("encode", seg_rows, n_seg, d_out);
  if (st != SFFN_OK) return st;
  REQUIRE(rec_bytes % 16 == 0 && (size_t)rec_bytes >= sparse_ffn_tier_record_bytes(d_out, n_seg),
          SFFN_EINVAL, "encode: rec_bytes=%d must be a multiple of 16 and >= %zu", rec_bytes,
          sparse_ffn_tier_record_bytes(d_out, n_seg));
  REQUIRE(aligned(Wt, 16) && aligned(mid_rec, 16), SFFN_EINVAL, "encode: pointers must be 16-byte aligned");
  if (n_in == 0) return ok();
  int b[5] = {0, 0, 0, 0, 0};
  for (int i = 0; i <= n_seg; ++i) b[i] = seg_rows[i];
  return from_hip(sffn::launch_encode_tiers(Wt, ld_w, n_in, d_out, b, n_seg, mid_rec, rec_bytes,
                                            (hipStream_t)stream),
                  "encode launch");
}

sffn_status sparse_ffn_tiered_gemv(const uint16_t* Wt, int ld_w, const uint8_t* mid_rec,
                                   int rec_bytes, const int32_t* seg_rows, int n_seg, int n_in,
                                   int d_out, const float* x, const int32_t* idx_top,
                                   const int32_t* cnt_top, int k_top_max, const int32_t* idx_mid,
                                   const int32_t* cnt_mid, int k_mid_max, float* y, int accumulate,
                                   void* workspace, size_t ws_bytes, void* stream) {
  REQUIRE(Wt && mid_rec && x && y, SFFN_EINVAL, "tiered: Wt, mid_rec, x and y must be non-null");
  REQUIRE(n_in >= 1 && d_out >= 64 && d_out % 64 == 0, SFFN_EINVAL,
          "tiered: need n_in >= 1 and d_out a positive multiple of 64 (d_out=%d)", d_out);
  REQUIRE(ld_w >= d_out && ld_w % 8 == 0, SFFN_EINVAL, "tiered: ld_w=%d must be >= d_out, %% 8",
          ld_w);
  sffn_status st = check_segments("tiered", seg_rows, n_seg, d_out);
  if (st != SFFN_OK) return st;
  REQUIRE(rec_bytes % 16 == 0 && (size_t)rec_bytes >= sparse_ffn_tier_record_bytes(d_out, n_seg),
          SFFN_EINVAL, "tiered: rec_bytes=%d must be a multiple of 16 and >= %zu", rec_bytes,
          sparse_ffn_tier_record_bytes(d_out, n_seg));
  REQUIRE(k_top_max >= 0 && k_top_max <= n_in && k_mid_max >= 0 && k_mid_max <= n_in, SFFN_EINVAL,
          "tiered: k_top_max=%d / k_mid_max=%d outside [0, n_in=%d]", k_top_max, k_mid_max, n_in);
  if (k_top_max > 0) REQUIRE(idx_top && cnt_top, SFFN_EINVAL, "tiered: top list needs idx and count");
  if (k_mid_max > 0) REQUIRE(idx_mid && cnt_mid, SFFN_EINVAL, "tiered: mid list needs idx and count");
  REQUIRE(aligned(Wt, 16) && aligned(mid_rec, 16) && aligned(y, 16) && aligned(x, 4), SFFN_EINVAL,
          "tiered: Wt/mid_rec/y must be 16-byte aligned, x 4-byte aligned");
  const size_t need = sffn::workspace_bytes(1, k_top_max + k_mid_max, d_out);
  REQUIRE(workspace != nullptr && ws_bytes >= need, SFFN_EWORKSPACE,
          "tiered: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  REQUIRE(aligned(workspace, 256), SFFN_EINVAL, "tiered: workspace must be 256-byte aligned");
  sffn::TierArgs a{};
  a.Wt = Wt; a.ld_w = ld_w; a.rec = mid_rec; a.rec_bytes = rec_bytes;
  for (int i = 0; i <= n_seg; ++i) a.seg_bounds[i] = seg_rows[i];
  a.n_seg = n_seg; a.n_in = n_in; a.d_out = d_out; a.x = x;
  a.idx_top = idx_top; a.cnt_top = cnt_top; a.k_top_max = k_top_max;
  a.idx_mid = idx_mid; a.cnt_mid = cnt_mid; a.k_mid_max = k_mid_max;
  a.y = y; a.accumulate = accumulate ? 1 : 0; a.ws = workspace; a.ws_bytes = ws_bytes;
  if (k_top_max > 0)
    DEBUG_CHECK_LIST("tiered (top)", 0, idx_top, cnt_top, k_top_max, n_in, true, (hipStream_t)stream);
  if (k_mid_max > 0)
    DEBUG_CHECK_LIST("tiered (mid)", 1, idx_mid, cnt_mid, k_mid_max, n_in, true, (hipStream_t)stream);
  return from_hip(sffn::launch_tiered(a, (hipStream_t)stream), "tiered launch");
}

sffn_status sparse_ffn_tiered_gemv_keyed(const uint16_t* Wt, int ld_w, const uint8_t* mid_rec,
                                         int rec_bytes, const int32_t* seg_rows, int n_seg,
                                         int n_in, int d_out, const float* x, const void* keys,
                                         int key_type, const uint32_t* thr_top, const uint32_t* thr,
                                         int k_top_max, int k_mid_max, float* y, int accumulate,
                                         void* workspace, size_t ws_bytes, void* stream) {
  REQUIRE(Wt && mid_rec && x && y, SFFN_EINVAL,
          "tiered_keyed: Wt, mid_rec, x and y must be non-null");
  REQUIRE(n_in >= 1 && d_out >= 64 && d_out % 64 == 0, SFFN_EINVAL,
          "tiered_keyed: need n_in >= 1 and d_out a positive multiple of 64 (d_out=%d)", d_out);
  REQUIRE(n_in <= 4096 * (sffn::kMaxSplit / 2), SFFN_EUNSUPPORTED,
          "tiered_keyed: n_in=%d above %d", n_in, 4096 * (sffn::kMaxSplit / 2));
  REQUIRE(ld_w >= d_out && ld_w % 8 == 0, SFFN_EINVAL,
          "tiered_keyed: ld_w=%d must be >= d_out, %% 8", ld_w);
  sffn_status st = check_segments("tiered_keyed", seg_rows, n_seg, d_out);
  if (st != SFFN_OK) return st;
  REQUIRE(rec_bytes % 16 == 0 && (size_t)rec_bytes >= sparse_ffn_tier_record_bytes(d_out, n_seg),
          SFFN_EINVAL, "tiered_keyed: rec_bytes=%d must be a multiple of 16 and >= %zu", rec_bytes,
          sparse_ffn_tier_record_bytes(d_out, n_seg));
  REQUIRE(keys != nullptr && aligned(keys, 4), SFFN_EINVAL,
          "tiered_keyed: keys must be non-null and 4-byte aligned");
  REQUIRE(key_type >= 0 && key_type <= 2, SFFN_EINVAL, "tiered_keyed: unknown key type %d",
          key_type);
  REQUIRE(thr_top && thr && aligned(thr_top, 8) && aligned(thr, 8), SFFN_EINVAL,
          "tiered_keyed: thr_top and thr must be non-null and 8-byte aligned");
  REQUIRE(k_top_max >= 0 && k_top_max <= n_in && k_mid_max >= 0 && k_mid_max <= n_in, SFFN_EINVAL,
          "tiered_keyed: k_top_max=%d / k_mid_max=%d outside [0, n_in=%d]", k_top_max, k_mid_max,
          n_in);
  REQUIRE(aligned(Wt, 16) && aligned(mid_rec, 16) && aligned(y, 16) && aligned(x, 4), SFFN_EINVAL,
          "tiered_keyed: Wt/mid_rec/y must be 16-byte aligned, x 4-byte aligned");
  const size_t need = sffn::workspace_bytes(1, k_top_max + k_mid_max, d_out);
  REQUIRE(workspace != nullptr && ws_bytes >= need, SFFN_EWORKSPACE,
          "tiered_keyed: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  REQUIRE(aligned(workspace, 256), SFFN_EINVAL, "tiered_keyed: workspace must be 256-byte aligned");
  sffn::TierArgs a{};
  a.Wt = Wt; a.ld_w = ld_w; a.rec = mid_rec; a.rec_bytes = rec_bytes;
  for (int i = 0; i <= n_seg; ++i) a.seg_bounds[i] = seg_rows[i];
  a.n_seg = n_seg; a.n_in = n_in; a.d_out = d_out; a.x = x;
  a.k_top_max = k_top_max; a.k_mid_max = k_mid_max;
  a.y = y; a.accumulate = accumulate ? 1 : 0; a.ws = workspace; a.ws_bytes = ws_bytes;
  a.keys = keys; a.key_type = key_type; a.thr_top = thr_top; a.thr = thr;
  return from_hip(sffn::launch_tiered(a, (hipStream_t)stream), "tiered_keyed launch");
}

sffn_status sparse_ffn_gemv_keyed(const uint16_t* W, int n_rows, int d, int ld_w, const float* in,
                                  const void* keys, int key_type, const uint32_t* thr, int k_max,
                                  const float* alpha, float* out, int accumulate, void* workspace,
                                  size_t ws_bytes, void* stream) {
  REQUIRE(W != nullptr && aligned(W, 16), SFFN_EINVAL,
          "gemv_keyed: W must be non-null and 16-byte aligned");
  REQUIRE(in != nullptr && aligned(in, 16), SFFN_EINVAL,
          "gemv_keyed: in must be non-null and 16-byte aligned");
  REQUIRE(out != nullptr && aligned(out, 16), SFFN_EINVAL,
          "gemv_keyed: out must be non-null and 16-byte aligned");
  REQUIRE(keys != nullptr && aligned(keys, 4), SFFN_EINVAL,
          "gemv_keyed: keys must be non-null and 4-byte aligned");
  REQUIRE(key_type >= 0 && key_type <= 2, SFFN_EINVAL, "gemv_keyed: unknown key type %d", key_type);
  REQUIRE(thr != nullptr && aligned(thr, 8), SFFN_EINVAL,
          "gemv_keyed: thr must be non-null and 8-byte aligned");
  REQUIRE(n_rows >= 1, SFFN_EINVAL, "gemv_keyed: n_rows=%d must be >= 1", n_rows);
  REQUIRE(d >= 8 && d % 8 == 0, SFFN_EINVAL, "gemv_keyed: d=%d must be a multiple of 8, >= 8", d);
  REQUIRE(ld_w >= d && ld_w % 8 == 0, SFFN_EINVAL, "gemv_keyed: ld_w=%d must be >= d, %% 8 == 0",
          ld_w);
  REQUIRE(k_max >= 0 && k_max <= n_rows, SFFN_EINVAL, "gemv_keyed: k_max=%d outside [0, n_rows=%d]",
          k_max, n_rows);
  if (alpha) REQUIRE(aligned(alpha, 4), SFFN_EINVAL, "gemv_keyed: alpha misaligned");
  const int col_tiles = (d + sffn::kTileCols - 1) / sffn::kTileCols;
  REQUIRE(sffn::keyed_split(n_rows, k_max, col_tiles) <= sffn::kMaxSplit, SFFN_EUNSUPPORTED,
          "gemv_keyed: n_rows=%d needs more row chunks than the reduction takes", n_rows);
  const size_t need = sffn::workspace_bytes(1, k_max, d);
  REQUIRE(workspace != nullptr && ws_bytes >= need, SFFN_EWORKSPACE,
          "gemv_keyed: workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  REQUIRE(aligned(workspace, 256), SFFN_EINVAL, "gemv_keyed: workspace must be 256-byte aligned");
  sffn::AxpyArgs a{W, n_rows, d, ld_w, in, 1, n_rows, nullptr, nullptr, k_max, 1,
                   nullptr, 0, alpha, out, d, accumulate ? 1 : 0, workspace, ws_bytes, 0, 0};
  return from_hip(sffn::launch_axpy_keyed(a, keys, key_type, thr, (hipStream_t)stream),
                  "gemv_keyed launch");
}

sffn_status sparse_ffn_gemv_noalloc(int op, const uint16_t* W0, const uint16_t* W1, int n_rows,
                                    int d, int ld_w, const float* in, int batch, int ld_in,
                                    const int32_t* idx, const int32_t* count, int k_max, int group,
                                    const uint8_t* row_mask, int ld_mask, float tau_scale,
                                    float rms_eps, const float* aux, int ld_aux, const float* alpha,
                                    float* out, uint32_t* key_out, int ld_out, int accumulate,
                                    void* stream) {
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if ((op & ~(SFFN_PACKED | SFFN_MASKED_ROWS)) == SFFN_OP_AXPY) {
    // the size check needs no GPU: sizes beyond the array are rejected first
    REQUIRE(batch >= 1 && d >= 8 && n_rows >= 0 && k_max >= 0 && group >= 1, SFFN_EINVAL,
            "gemv_noalloc: bad shape (batch=%d d=%d n_rows=%d k_max=%d group=%d)", batch, d,
            n_rows, k_max, group);
    const long items = idx ? (long)k_max * group : (long)n_rows;
    REQUIRE(items <= n_rows, SFFN_EINVAL, "gemv_noalloc: k_max=%d * group=%d exceeds n_rows=%d",
            k_max, group, n_rows);
    const size_t need = sffn::workspace_bytes(batch, (int)items, d);
    REQUIRE(need <= kScratchBytes, SFFN_EWORKSPACE,
            "gemv_noalloc: this product needs %zu bytes of scratch, above the %zu-byte static "
            "array (use sparse_ffn_gemv with a workspace)", need, kScratchBytes);
    const sffn_status st = current_scratch(&ws);
    if (st != SFFN_OK) return st;
    ws_bytes = kScratchBytes;
  }
  // row ops use no scratch; everything else (validation, kernels) is
  // sparse_ffn_gemv's, which allocates nothing
  return sparse_ffn_gemv(op, W0, W1, n_rows, d, ld_w, in, batch, ld_in, idx, count, k_max, group,
                         row_mask, ld_mask, tau_scale, rms_eps, aux, ld_aux, alpha, out, key_out,
                         ld_out, accumulate, ws, ws_bytes, stream);
}

}  // extern "C"
