// Gathered down projection at batch 1:
//   y[o] = (accumulate ? y[o] : 0) + alpha * sum_{processed rows n} m_n a_n W^T[n][o]
// reading only the selected rows of W_down^T (SelectInfer §5 computes only
// the selected neurons; LeanStream "Permutation-Invariant Execution": the
// output is a sum over hidden neurons, so any row order gives the same y up
// to fp32 rounding).
//
// Grid = (512-column tiles) x (KS row chunks).  A 1024-thread workgroup owns
// one column tile and one contiguous chunk of the compacted row list; wave w
// takes rows w, w+16, ...; lane l owns columns 8l..8l+7 of the tile and
// reads them with one 16-byte load per row (1 KiB per wave instruction).
// Waves are summed in LDS, the chunk's partial goes to the workspace, and
// the last workgroup to finish a column tile sums all chunks in chunk order
// (fixed order: the result is bitwise reproducible) and writes y.
#include "sffn_splitk.h"

namespace sffn {

__global__ __launch_bounds__(1024) void axpy_b1_kernel(AxpyArgs a, int KS) {
  __shared__ float4 red[kWaves][kTileCols / 4];
  __shared__ int last_flag;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int col = tile * kTileCols + 8 * lane;
  const bool col_ok = col < a.d;

  const int n_items = item_count(a.idx, a.count, a.k_max, a.group, a.n_rows);
  const int chunk = (n_items + KS - 1) / KS;
  const int k0 = ks * chunk;
  const int k1 = min(n_items, k0 + chunk);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;
  for (int kb = k0 + w; kb < k1; kb += kWaves * U) {
    int row[U];
    float av[U];
    uint4 wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = kb + kWaves * u;
      const bool ok = it < k1;
      row[u] = ok ? item_row(a.idx, a.group, it) : 0;
      float v = 0.f;
      if (ok) {
        v = a.in[row[u]];
        if (a.row_mask && !a.row_mask[row[u]]) v = 0.f;
      }
      av[u] = v;
      wv[u] = (ok && col_ok) ? *reinterpret_cast<const uint4*>(a.W + (size_t)row[u] * a.ld_w + col)
                             : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[8];
      unpack8(wv[u], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(av[u], f[e], acc[e]);
    }
  }

  const float part = wg_reduce_cols(red, acc);
  uint32_t* counters = reinterpret_cast<uint32_t*>(a.ws);
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kCounterBytes);
  splitk_finish(red, &last_flag, part, partials, counters + tile, KS, ks, tile, a.d, a.alpha,
                a.out, a.accumulate);
}

int pick_split_b1(long items, int col_tiles) {
  // about two 16-wave workgroups per CU, at least one row per wave
  long ks = (512 + col_tiles - 1) / col_tiles;
  const long max_by_rows = (items + kWaves - 1) / kWaves;
  if (ks > max_by_rows) ks = max_by_rows;
  if (ks > kMaxSplit) ks = kMaxSplit;
  if (ks < 1) ks = 1;
  return (int)ks;
}

hipError_t launch_axpy_b1(const AxpyArgs& a, hipStream_t s) {
  const int col_tiles = (a.d + kTileCols - 1) / kTileCols;
  const long items = a.idx ? (long)a.k_max * a.group : (long)a.n_rows;
  const int KS = pick_split_b1(items, col_tiles);
  hipLaunchKernelGGL(axpy_b1_kernel, dim3(col_tiles, KS), dim3(1024), 0, s, a, KS);
  return hipGetLastError();
}

}  // namespace sffn
