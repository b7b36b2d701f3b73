// Split-K pieces shared by the gathered products (plain, tiered, batched):
// row-list expansion, the in-workgroup column reduction, streaming loads and
// the ordered reduction of per-chunk partials.  Internal to libsparse_ffn.so.
//
// A gathered product splits its row list into KS chunks; each chunk's
// workgroups write fp32 partials [KS][M][d] to the workspace and a second
// kernel sums them in chunk order (fixed order: bitwise reproducible; no
// float atomics, no cross-workgroup fences inside a kernel).
#pragma once

#include "sffn_device.h"

namespace sffn {

constexpr int kTileCols = 512;
constexpr int kWaves = 16;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte nontemporal (streaming) load of weights that are read once.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t load_stream4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

__device__ __forceinline__ int item_count(const int32_t* idx, const int32_t* count, int k_max,
                                          int group, int n_rows) {
  if (!idx) return n_rows;
  int c = *count;
  c = c < k_max ? c : k_max;
  return (c > 0 ? c : 0) * group;
}

__device__ __forceinline__ int item_row(const int32_t* idx, int group, int it) {
  if (!idx) return it;
  const int q = it / group;
  return idx[q] * group + (it - q * group);
}

// Sum the 16 waves' 8-column partials held in `acc` (lane owns columns
// 8*lane..8*lane+7) in wave order; threads 0..511 return their column's sum.
__device__ __forceinline__ float wg_reduce_cols(float4 (*red)[kTileCols / 4], const float (&acc)[8]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  red[w][2 * lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  red[w][2 * lane + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x < kTileCols) {
    const float* r = reinterpret_cast<const float*>(red);
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s += r[ww * kTileCols + threadIdx.x];
  }
  return s;
}

// Launch the ordered reduction: out[m][c] = (accumulate ? out[m][c] : 0) +
// alpha[m] * sum_{k < KS} partials[k][m][c]   (partials [KS][Mp][d]).
hipError_t launch_splitk_reduce(const float* partials, int KS, int M, int Mp, int d,
                                const float* alpha, float* out, int ld_out, int accumulate,
                                hipStream_t s);

}  // namespace sffn
