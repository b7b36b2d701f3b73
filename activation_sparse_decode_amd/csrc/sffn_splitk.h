// Split-K pieces shared by the batch-1 gathered products (plain and tiered):
// row-list expansion, the in-workgroup column reduction, and the
// last-workgroup-reduces epilogue.  Internal to libsparse_ffn.so.
#pragma once

#include "sffn_device.h"

namespace sffn {

constexpr int kTileCols = 512;
constexpr int kWaves = 16;

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
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  red[w][2 * lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  red[w][2 * lane + 1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x < kTileCols) {
    const float* r = reinterpret_cast<const float*>(red);
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s += r[ww * kTileCols + threadIdx.x];
  }
  __syncthreads();
  return s;
}

// Split-K epilogue shared by the batch-1 kernels: publish this chunk's
// partial; the last chunk of the tile reduces all chunks in order.
__device__ inline void splitk_finish(float4 (*red)[kTileCols / 4], int* last_flag, float part,
                              float* partials, uint32_t* counter, int KS, int ks, int tile,
                              int d, const float* alpha, float* out, int accumulate) {
  const int c = tile * kTileCols + (int)threadIdx.x;
  if (threadIdx.x < kTileCols && c < d) partials[(size_t)ks * d + c] = part;
  // One agent-scope fence per workgroup (release of the whole group's
  // partial, made cumulative by the barrier), then the arrival counter.
  __syncthreads();
  if (threadIdx.x == 0) {
    __threadfence();
    const unsigned prev = atomicAdd(counter, 1u);
    *last_flag = (prev == (unsigned)(KS - 1));
    if (*last_flag) __threadfence();   // acquire: the other chunks' partials
  }
  __syncthreads();
  if (!*last_flag) return;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = tile * kTileCols + 8 * lane;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col < d) {
    for (int kk = w; kk < KS; kk += kWaves) {
      const float4 p = *reinterpret_cast<const float4*>(partials + (size_t)kk * d + col);
      const float4 q = *reinterpret_cast<const float4*>(partials + (size_t)kk * d + col + 4);
      acc[0] += p.x; acc[1] += p.y; acc[2] += p.z; acc[3] += p.w;
      acc[4] += q.x; acc[5] += q.y; acc[6] += q.z; acc[7] += q.w;
    }
  }
  const float total = wg_reduce_cols(red, acc);
  if (threadIdx.x < kTileCols && c < d) {
    const float al = alpha ? *alpha : 1.f;
    const float base = accumulate ? out[c] : 0.f;
    out[c] = base + al * total;
  }
  if (threadIdx.x == 0) *counter = 0u;
}

}  // namespace sffn
