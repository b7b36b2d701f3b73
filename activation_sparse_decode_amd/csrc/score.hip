// Scores that feed the selection.
//  SUM_ABS      SelectInfer §3, Eq (1): s_n = sum over tokens of |a_n(t)|.
//               One thread per neuron adds the tokens in order in fp32 (one
//               rounding per add), so the result is a fixed function of the
//               inputs; loads are coalesced across neurons.
//  CLUSTER_MAX  kappa_c = max over the cluster's rows of the magnitude key
//               (PowerInfer-2 guide, "Neuron Cluster Decomposition").  Max
//               is order-free, so the result is exact.
//  SOFTMAX_PICKED  mixing weights of the picked entries of a row (the two
//               routed experts of the MoE layer).
// Row norms of a bf16 matrix (offline): ||W[r]||_2 of each row of W^T, the
// weight norm of input channel r that WiSparse's weight-aware saliency
// multiplies with the activation magnitude.  A wave per row; lane l adds
// the squares of chunks l, l+64, ... in order, then the wave sum.
#include "sffn_device.h"

namespace sffn {

__global__ __launch_bounds__(256) void score_sum_abs_kernel(const float* __restrict__ in, int T,
                                                            int n, int ld, int accumulate,
                                                            float* __restrict__ s) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = accumulate ? s[i] : 0.f;
  for (int t = 0; t < T; ++t) acc = acc + fabsf(in[(size_t)t * ld + i]);
  s[i] = acc;
}

__global__ __launch_bounds__(256) void score_cluster_max_kernel(const float* __restrict__ in, int T,
                                                                int n, int ld, int cluster,
                                                                uint32_t* __restrict__ out) {
  const int nc = n / cluster;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)nc * T) return;
  const int t = (int)(i / nc), c = (int)(i - (long)t * nc);
  const float* p = in + (size_t)t * ld + (size_t)c * cluster;
  uint32_t m = 0u;
  for (int r = 0; r < cluster; ++r) {
    const uint32_t k = key_abs(p[r]);
    m = k > m ? k : m;
  }
  out[(size_t)t * nc + c] = m;
}

__global__ __launch_bounds__(256) void score_softmax_picked_kernel(const float* __restrict__ in,
                                                                   int T, int ld,
                                                                   const int32_t* __restrict__ picked,
                                                                   int k, float* __restrict__ out) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const float* v = in + (size_t)t * ld;
  const int32_t* p = picked + (size_t)t * k;
  float m = v[p[0]];
  for (int j = 1; j < k; ++j) m = fmaxf(m, v[p[j]]);
  float z = 0.f;
  for (int j = 0; j < k; ++j) z += expf(v[p[j]] - m);
  for (int j = 0; j < k; ++j) out[(size_t)t * k + j] = expf(v[p[j]] - m) / z;
}

__global__ __launch_bounds__(256) void row_norms_kernel(const uint16_t* __restrict__ W, int n_rows,
                                                        int d, int ld_w, float* __restrict__ out) {
  const int r = blockIdx.x * 4 + wave_id();
  if (r >= n_rows) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* w = W + (size_t)r * ld_w;
  float s = 0.f;
  for (int c = lane; c < (d >> 3); c += 64) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(w + 8 * c), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(f[e], f[e], s);
  }
  s = wave_sum(s);
  if (lane == 0) out[r] = sqrtf(s);
}

hipError_t launch_row_norms(const uint16_t* W, int n_rows, int d, int ld_w, float* out,
                            hipStream_t s) {
  hipLaunchKernelGGL(row_norms_kernel, dim3((n_rows + 3) / 4), dim3(256), 0, s, W, n_rows, d, ld_w,
                     out);
  return hipGetLastError();
}

hipError_t launch_score(int mode, const float* in, int T, int n, int ld, int cluster,
                        int accumulate, const int32_t* picked, int k, void* out, hipStream_t s) {
  if (mode == 0) {
    hipLaunchKernelGGL(score_sum_abs_kernel, dim3((n + 255) / 256), dim3(256), 0, s, in, T, n, ld,
                       accumulate, reinterpret_cast<float*>(out));
  } else if (mode == 1) {
    const long total = (long)(n / cluster) * T;
    hipLaunchKernelGGL(score_cluster_max_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       0, s, in, T, n, ld, cluster, reinterpret_cast<uint32_t*>(out));
  } else {
    hipLaunchKernelGGL(score_softmax_picked_kernel, dim3((T + 255) / 256), dim3(256), 0, s, in, T,
                       ld, picked, k, reinterpret_cast<float*>(out));
  }
  return hipGetLastError();
}

}  // namespace sffn
