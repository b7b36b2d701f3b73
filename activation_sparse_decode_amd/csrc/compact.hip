// One-time physical compaction of a selected neuron set.
//
// LeanStream ("Permutation-Invariant Execution") treats a subset of FFN
// neurons as one contiguous dense matrix, since the FFN output is a sum over
// neurons in any order; SelectInfer (§5) fixes the computed set U for the
// whole decode of a prompt.  Gathering U's weights once per prompt turns
// every decode step into dense, index-free streaming:
//  - rows:       out[i][:] = W[idx_i][:]     (gate / up rows of U)
//  - transposed: out[o][i] = W[idx_i][o]     (down rows of U laid out output-
//                major, so the down projection becomes one dot product per
//                output over the compacted activations); columns i >= k up
//                to ld_out are zero.
// The packed layouts of the batched MFMA kernels are built here too (a
// one-time re-layout of a weight matrix at load time).
// A 4-byte gather, dst[i] = src[idx_i], carries per-neuron values (scores,
// masks, keys) into the positions of a compacted subset: the index remap of
// a selectively loaded layer (SelectInfer §4), whose resident weights hold
// only the loaded neurons, in ascending order.
#include <algorithm>

#include "sffn_device.h"

namespace sffn {

__global__ __launch_bounds__(256) void compact_rows_kernel(const uint16_t* __restrict__ W, int ld_w,
                                                           int d, const int32_t* __restrict__ idx,
                                                           int k, uint16_t* __restrict__ out,
                                                           int ld_out) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + wave_id();
  if (i >= k) return;
  const uint16_t* src = W + (size_t)idx[i] * ld_w;
  uint16_t* dst = out + (size_t)i * ld_out;
  for (int c = lane; c < (d >> 3); c += 64)
    *reinterpret_cast<uint4*>(dst + 8 * c) = *reinterpret_cast<const uint4*>(src + 8 * c);
}

// 64 (neurons) x 64 (outputs) tile through LDS.
__global__ __launch_bounds__(256) void compact_cols_kernel(const uint16_t* __restrict__ W, int ld_w,
                                                           int d, const int32_t* __restrict__ idx,
                                                           int k, uint16_t* __restrict__ out,
                                                           int ld_out) {
  __shared__ uint16_t T[64][66];
  const int t = threadIdx.x;
  const int i0 = blockIdx.x * 64, o0 = blockIdx.y * 64;
  {
    const int r = t >> 2, q = t & 3;          // neuron i0+r, outputs o0+16q .. +16
    const int i = i0 + r, o = o0 + 16 * q;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (i < k) {
      const uint16_t* src = W + (size_t)idx[i] * ld_w + o;
      if (o < d) v0 = *reinterpret_cast<const uint4*>(src);
      if (o + 8 < d) v1 = *reinterpret_cast<const uint4*>(src + 8);
    }
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      T[r][16 * q + 2 * e] = (uint16_t)(w[e] & 0xFFFFu);
      T[r][16 * q + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  {
    const int r = t >> 2, q = t & 3;          // output o0+r, neurons i0+16q .. +16
    const int o = o0 + r, i = i0 + 16 * q;
    if (o >= d) return;
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      w[e] = (uint32_t)T[16 * q + 2 * e][r] | ((uint32_t)T[16 * q + 2 * e + 1][r] << 16);
    uint16_t* dst = out + (size_t)o * ld_out + i;
    if (i + 8 <= ld_out) *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    if (i + 16 <= ld_out) *reinterpret_cast<uint4*>(dst + 8) = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// dst[i] = src[idx[i]] for i < min(*count, k_max) (k_max without a count);
// an index outside [0, n_src) reads the nearest valid element.
__global__ __launch_bounds__(256) void gather32_kernel(const uint32_t* __restrict__ src, int n_src,
                                                       const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ count, int k_max,
                                                       uint32_t* __restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int k = count ? min(max(*count, 0), k_max) : k_max;
  if (i >= k) return;
  dst[i] = src[min(max(idx[i], 0), n_src - 1)];
}

hipError_t launch_gather32(const uint32_t* src, int n_src, const int32_t* idx,
                           const int32_t* count, int k_max, uint32_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(gather32_kernel, dim3((k_max + 255) / 256), dim3(256), 0, s, src, n_src, idx,
                     count, k_max, dst);
  return hipGetLastError();
}

// Packed layouts of the batched kernels (see sffn_device.h), one 16-byte
// output unit per thread: each thread reads the 8 weights its unit holds
// from the row-major source (zeros for padding rows) and stores them, so
// the stores are contiguous.
__global__ __launch_bounds__(256) void pack_row_tiles_kernel(const uint16_t* __restrict__ W,
                                                             int n_rows, int d, int ld_w,
                                                             uint16_t* __restrict__ out,
                                                             size_t units) {
  const int cpr = d >> 7;   // 128-wide chunks per row
  for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < units;
       u += (size_t)gridDim.x * blockDim.x) {
    // u = ((tile * cpr + chunk) * 16 + row in tile) * 16 + unit in chunk
    const int q = (int)(u & 15);
    const int rr = (int)((u >> 4) & 15);
    const size_t tc = u >> 8;
    const int c = (int)(tc % cpr);
    const size_t r = (tc / cpr) * 16 + rr;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < (size_t)n_rows) v = *reinterpret_cast<const uint4*>(W + r * ld_w + 128 * c + 8 * q);
    *reinterpret_cast<uint4*>(out + 8 * u) = v;
  }
}

__global__ __launch_bounds__(256) void pack_col_panels_kernel(const uint16_t* __restrict__ W,
                                                              int n_rows, int ld_w,
                                                              uint16_t* __restrict__ out,
                                                              size_t units) {
  for (size_t u = blockIdx.x * (size_t)blockDim.x + threadIdx.x; u < units;
       u += (size_t)gridDim.x * blockDim.x) {
    // u = (panel * n_rows + row) * 32 + unit in panel row
    const int q = (int)(u & 31);
    const size_t pr = u >> 5;
    const size_t r = pr % (size_t)n_rows;
    const size_t p = pr / (size_t)n_rows;
    *reinterpret_cast<uint4*>(out + 8 * u) =
        *reinterpret_cast<const uint4*>(W + r * ld_w + 256 * p + 8 * q);
  }
}

size_t packed_elems(int n_rows, int d, int layout) {
  if (n_rows < 0 || d <= 0) return 0;
  if (layout == kLayoutRowTiles && d % 128 == 0) return ((size_t)n_rows + 15) / 16 * 16 * d;
  if (layout == kLayoutColPanels && d % 256 == 0) return (size_t)n_rows * d;
  return 0;
}

hipError_t launch_pack(const uint16_t* W, int n_rows, int d, int ld_w, int layout, uint16_t* out,
                       hipStream_t s) {
  const size_t units = packed_elems(n_rows, d, layout) / 8;
  if (units == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((units + 255) / 256, 8192);
  if (layout == kLayoutRowTiles)
    hipLaunchKernelGGL(pack_row_tiles_kernel, dim3(blocks), dim3(256), 0, s, W, n_rows, d, ld_w,
                       out, units);
  else
    hipLaunchKernelGGL(pack_col_panels_kernel, dim3(blocks), dim3(256), 0, s, W, n_rows, ld_w, out,
                       units);
  return hipGetLastError();
}

hipError_t launch_compact(const uint16_t* W, int ld_w, int d, const int32_t* idx, int k,
                          int transpose, uint16_t* out, int ld_out, hipStream_t s) {
  if (!transpose) {
    if (k == 0) return hipSuccess;
    hipLaunchKernelGGL(compact_rows_kernel, dim3((k + 3) / 4), dim3(256), 0, s, W, ld_w, d, idx, k,
                       out, ld_out);
  } else {
    dim3 grid((ld_out + 63) / 64, (d + 63) / 64);
    hipLaunchKernelGGL(compact_cols_kernel, grid, dim3(256), 0, s, W, ld_w, d, idx, k, out,
                       ld_out);
  }
  return hipGetLastError();
}

}  // namespace sffn
