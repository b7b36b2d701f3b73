// Gathered down projection at batch 1:
//   y[o] = (accumulate ? y[o] : 0) + alpha * sum_{processed rows n} m_n a_n W^T[n][o]
// reading only the selected rows of W_down^T (SelectInfer §5 computes only
// the selected neurons; LeanStream "Permutation-Invariant Execution": the
// output is a sum over hidden neurons, so any row order gives the same y up
// to fp32 rounding).
//
// Kernel 1, grid = (512-column tiles) x (KS row chunks): a 1024-thread
// workgroup owns one column tile and one contiguous chunk of the compacted
// row list; wave w takes rows w, w+16, ...; lane l owns columns 8l..8l+7 of
// the tile and streams them with one 16-byte nontemporal load per row
// (1 KiB per wave instruction), four or eight rows in flight per lane.  Waves are summed in LDS and the chunk's
// partial row goes to the workspace.  Kernel 2 sums the KS partials in chunk
// order and applies alpha / accumulate.
#include <algorithm>
#include <type_traits>

#include "sffn_splitk.h"

namespace sffn {

__device__ __forceinline__ uint32_t lanes_below_u64(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Adds this wave's rows of the chunk [k0, k1) of a row list to acc: wave w
// takes items k0 + w + kWaves * u.  Their rows, activations and masks are
// fetched with one vector load per lane (lane l: item u = ub + l), then
// broadcast with readlane, so the weight loads of all of the wave's rows are
// issued back to back without waiting on indices.
__device__ __forceinline__ void axpy_chunk(const uint16_t* W, int ld_w, const float* in,
                                           const int32_t* idx, int group, const uint8_t* row_mask,
                                           int k0, int k1, int colc, float (&acc)[8]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int nu = k1 - k0 > w ? (k1 - k0 - w + kWaves - 1) / kWaves : 0;
  for (int ub = 0; ub < nu; ub += 64) {
    const bool ok = ub + lane < nu;
    const int it = k0 + w + kWaves * (ok ? ub + lane : 0);
    const int r = item_row(idx, group, it);
    const int nb = min(64, nu - ub);
    // Every load of a batch is issued (a padding slot past the wave's last
    // row re-reads its first row with weight 0): no branch around a load, so
    // nothing waits between them.  The activations are gathered after the
    // batch's weights were requested (r is a valid row for every lane), so
    // their wait is the batch's wait.
    auto batch = [&](int u, auto width) {
      constexpr int U = decltype(width)::value;
      uint4 wv[U];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int rr = __builtin_amdgcn_readlane(r, u + uu < nb ? u + uu : 0);
        wv[uu] = load_stream16(W + (size_t)rr * ld_w + colc);
      }
      float v = in[r];
      if (row_mask && !row_mask[r]) v = 0.f;
      const float av = ok ? v : 0.f;
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int src = u + uu < nb ? u + uu : 0;
        const float au = u + uu < nb ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(av), src)) : 0.f;
        float f[8];
        unpack8(wv[uu], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(au, f[e], acc[e]);
      }
    };
    // eight rows in flight per lane while at least eight remain, then four
    int u = 0;
    for (; u + 8 <= nb; u += 8) batch(u, std::integral_constant<int, 8>());
    for (; u < nb; u += 4) batch(u, std::integral_constant<int, 4>());
  }
}

__global__ __launch_bounds__(1024) void axpy_b1_kernel(AxpyArgs a, int KS, float* partials) {
  __shared__ float4 red[kWaves][kTileCols / 4];
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int col = tile * kTileCols + 8 * lane;
  const int colc = col < a.d ? col : 0;   // lanes past the last column re-read column 0 (discarded)

  const int n_items = item_count(a.idx, a.count, a.k_max, a.group, a.n_rows);
  const int chunk = (n_items + KS - 1) / KS;
  const int k0 = ks * chunk;
  const int k1 = min(n_items, k0 + chunk);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  axpy_chunk(a.W, a.ld_w, a.in, a.idx, a.group, a.row_mask, k0, k1, colc, acc);

  const float part = wg_reduce_cols(red, acc);
  const int c = tile * kTileCols + (int)threadIdx.x;
  if (threadIdx.x < kTileCols && c < a.d) partials[(size_t)ks * a.d + c] = part;
}

// Several row lists into one output: chunk ks belongs to the list l with
// ks_begin[l] <= ks < ks_begin[l+1]; its partial is scaled by alpha_l here,
// so the ordered reduction adds plain partials.
struct ListChunks { int ks_begin[kMaxLists + 1]; };

__global__ __launch_bounds__(1024) void axpy_lists_kernel(AxpyListsArgs a, ListChunks lc,
                                                          float* partials) {
  __shared__ float4 red[kWaves][kTileCols / 4];
  const int lane = threadIdx.x & 63;
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int col = tile * kTileCols + 8 * lane;
  const int colc = col < a.d ? col : 0;   // lanes past the last column re-read column 0 (discarded)
  int l = 0;
#pragma unroll
  for (int i = 1; i < kMaxLists; ++i) l += (i < a.n && ks >= lc.ks_begin[i]) ? 1 : 0;
  const AxpyList L = a.l[l];
  const int KS = lc.ks_begin[l + 1] - lc.ks_begin[l];
  const int n_items = item_count(L.idx, L.count, L.k_max, a.group, 0);
  const int chunk = (n_items + KS - 1) / KS;
  const int k0 = (ks - lc.ks_begin[l]) * chunk;
  const int k1 = min(n_items, k0 + chunk);
  const float al = L.alpha ? *L.alpha : 1.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  axpy_chunk(L.W, a.ld_w, L.in, L.idx, a.group, nullptr, k0, k1, colc, acc);

  const float part = wg_reduce_cols(red, acc);
  const int c = tile * kTileCols + (int)threadIdx.x;
  if (threadIdx.x < kTileCols && c < a.d) partials[(size_t)ks * a.d + c] = al * part;
}

// Ordered reduction of [KS][Mp][d] partials.  A 256-thread workgroup covers
// 64 columns of one token row: lane group g (16 lanes, one float4 each) sums
// the chunks g, g+16, ... with all of its loads issued before the first add
// (the reduction is latency-bound, not bandwidth-bound), then the 16 group
// sums are added in group order.  The order is fixed, so results are
// reproducible run to run.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partials,
                                                            int KS, int Mp, int d,
                                                            const float* __restrict__ alpha,
                                                            float* __restrict__ out, int ld_out,
                                                            int accumulate) {
  constexpr int kGroups = 16;
  constexpr int kPerGroup = kMaxSplit / kGroups;
  __shared__ float4 red[kGroups][16];
  const int q = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int m = blockIdx.y;
  const int c = blockIdx.x * 64 + 4 * q;
  const int cc = c < d ? c : 0;   // lanes past the last column re-read column 0 (discarded)
  // The values added to (with accumulate) and the scale are requested right
  // after the partials, so the epilogue does not wait for them (and the
  // scale's scalar load does not hold back the partials' requests).
  float* o = out + (size_t)m * ld_out + cc;   // 4-byte aligned (ld_out may be any stride)
  float4 v[kPerGroup];
#pragma unroll
  for (int i = 0; i < kPerGroup; ++i) {
    const int k = g + kGroups * i;
    v[i] = k < KS ? *reinterpret_cast<const float4*>(partials + ((size_t)k * Mp + m) * d + cc)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float prev[4] = {0.f, 0.f, 0.f, 0.f};
  if (accumulate) {
#pragma unroll
    for (int e = 0; e < 4; ++e) prev[e] = o[e];
  }
  asm volatile("" ::: "memory");
  const float al = alpha ? alpha[m] : 1.f;
  float4 s = v[0];
#pragma unroll
  for (int i = 1; i < kPerGroup; ++i) {
    s.x += v[i].x; s.y += v[i].y; s.z += v[i].z; s.w += v[i].w;
  }
  red[g][q] = s;
  __syncthreads();
  if (g != 0 || c >= d) return;
  float4 t = red[0][q];
#pragma unroll
  for (int gg = 1; gg < kGroups; ++gg) {
    const float4 r = red[gg][q];
    t.x += r.x; t.y += r.y; t.z += r.z; t.w += r.w;
  }
  const float tv[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = prev[e] + al * tv[e];
}

hipError_t launch_splitk_reduce(const float* partials, int KS, int M, int Mp, int d,
                                const float* alpha, float* out, int ld_out, int accumulate,
                                hipStream_t s) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((d + 63) / 64, M), dim3(256), 0, s, partials, KS,
                     Mp, d, alpha, out, ld_out, accumulate);
  return hipGetLastError();
}

int pick_split_b1(long items, int col_tiles) {
  // about four rows per wave (the loads a lane keeps in flight), within
  // 256..512 workgroups: every CU streams, and a device-side count far
  // below the launch bound `items` still leaves a few rows per wave.  The
  // upper bound rounds down: two 1024-thread workgroups fit a CU, so 512 is
  // one round, and a few workgroups past it would start only when the first
  // ones end (at 10 column tiles, 520 workgroups took 8% longer than 510)
  long ks = (items + 4 * kWaves - 1) / (4 * kWaves);
  const long min_ks = (256 + col_tiles - 1) / col_tiles;
  const long max_ks = std::max(1, 512 / col_tiles);
  if (ks < min_ks) ks = min_ks;
  if (ks > max_ks) ks = max_ks;
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
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes);
  hipLaunchKernelGGL(axpy_b1_kernel, dim3(col_tiles, KS), dim3(1024), 0, s, a, KS, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(partials, KS, 1, 1, a.d, a.alpha, a.out, a.d, a.accumulate, s);
}

hipError_t launch_axpy_lists(const AxpyListsArgs& a, hipStream_t s) {
  const int col_tiles = (a.d + kTileCols - 1) / kTileCols;
  long items = 0;
  for (int l = 0; l < a.n; ++l) items += (long)a.l[l].k_max * a.group;
  // the split one product of all the rows would take, shared out by the
  // lists' row bounds (every list with rows keeps at least one chunk)
  // (every list's rounding may add one chunk: keep the total within kMaxSplit)
  const int KS = std::min(pick_split_b1(items, col_tiles), kMaxSplit - a.n);
  ListChunks lc{};
  int ks = 0;
  for (int l = 0; l < a.n; ++l) {
    lc.ks_begin[l] = ks;
    const long li = (long)a.l[l].k_max * a.group;
    long k = items > 0 ? (long)((double)KS * (double)li / (double)items + 0.5) : 0;
    if (li > 0 && k < 1) k = 1;
    if (k > (li + kWaves - 1) / kWaves) k = (li + kWaves - 1) / kWaves;
    ks += (int)k;
  }
  for (int l = a.n; l <= kMaxLists; ++l) lc.ks_begin[l] = ks;
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes);
  if (ks > 0) {
    hipLaunchKernelGGL(axpy_lists_kernel, dim3(col_tiles, ks), dim3(1024), 0, s, a, lc, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // no rows at all: zero chunks, the reduction writes out (+)= 0
  return launch_splitk_reduce(partials, ks, 1, 1, a.d, nullptr, a.out, a.d, a.accumulate, s);
}


// ---------------------------------------------------------------- keyed rows
// The product over the rows a threshold selects, with no index list: chunk ks
// of the grid covers the neurons [ks c, min(n, (ks + 1) c)), c <= 1024, and
// wave w of the workgroup the w-th sixteenth of it (at most 64 neurons, one
// per lane).  Each lane tests its neuron's key against (T, I); the selected
// neurons of the wave, in index order, are sent to lanes 0, 1, ...
// (ds_permute to the lane's rank in the ballot), so lane q holds the wave's
// q-th row; the rows then stream as in the listed product, and the partials
// go to the same ordered reduction.
__device__ __forceinline__ uint32_t keyed_key(const void* keys, int key_type, int n) {
  const uint32_t b = reinterpret_cast<const uint32_t*>(keys)[n];
  if (key_type == 0) return b & 0x7FFFFFFFu;
  if (key_type == 1) return b;
  return key_signed(__uint_as_float(b));
}

__global__ __launch_bounds__(1024) void axpy_keyed_kernel(AxpyArgs a, const void* keys, int key_type,
                                                          const uint32_t* thr, int KS,
                                                          float* partials) {
  __shared__ float4 red[kWaves][kTileCols / 4];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int col = tile * kTileCols + 8 * lane;
  const int colc = col < a.d ? col : 0;   // lanes past the last column re-read column 0 (discarded)
  const int N = a.n_rows;
  const int chunk = (N + KS - 1) / KS;
  const int sub = (chunk + kWaves - 1) / kWaves;   // <= 64
  const int n0 = ks * chunk, n1 = min(N, n0 + chunk);
  const int s0 = n0 + w * sub, s1 = min(n1, s0 + sub);
  const uint32_t T = thr[0];
  const int I = (int)thr[1];

  const int nn = s0 + lane;
  const uint32_t kv = keyed_key(keys, key_type, min(nn, N - 1));   // clamped: no branch around a load
  const bool in = nn < s1 && (kv > T || (kv == T && nn <= I));
  const uint64_t m = __ballot(in);
  const int nb = (int)__popcll(m);
  // lane q receives the q-th selected neuron; the others send to lane 63,
  // which is a row slot only when all 64 are selected (then nobody else sends)
  const int got = __builtin_amdgcn_ds_permute((in ? (int)lanes_below_u64(m) : 63) << 2, nn);
  const int r = lane < nb ? got : min(s0, N - 1);   // a valid row for every lane

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (nb > 0) {
    const float av = lane < nb ? a.in[r] : 0.f;
    auto batch = [&](int u, auto width) {
      constexpr int U = decltype(width)::value;
      uint4 wv[U];
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const int rr = __builtin_amdgcn_readlane(r, u + uu < nb ? u + uu : 0);
        wv[uu] = load_stream16(a.W + (size_t)rr * a.ld_w + colc);
      }
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const float au = u + uu < nb
            ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(av), u + uu)) : 0.f;
        float f[8];
        unpack8(wv[uu], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(au, f[e], acc[e]);
      }
    };
    // eight rows in flight per lane while more than four remain, then four
    int u = 0;
    for (; nb - u > 4; u += 8) batch(u, std::integral_constant<int, 8>());
    if (u < nb) batch(u, std::integral_constant<int, 4>());
  }

  const float part = wg_reduce_cols(red, acc);
  const int c = tile * kTileCols + (int)threadIdx.x;
  if (threadIdx.x < kTileCols && c < a.d) partials[(size_t)ks * a.d + c] = part;
}

// Chunk count: the listed product's split for k_max rows, raised until a
// chunk fits 16 waves x 64 neurons.
int keyed_split(int n_rows, long k_max, int col_tiles) {
  const int KS = pick_split_b1(k_max, col_tiles);
  const int need = (n_rows + kWaves * 64 - 1) / (kWaves * 64);
  return std::max(KS, need);
}

hipError_t launch_axpy_keyed(const AxpyArgs& a, const void* keys, int key_type, const uint32_t* thr,
                             hipStream_t s) {
  const int col_tiles = (a.d + kTileCols - 1) / kTileCols;
  const int KS = keyed_split(a.n_rows, a.k_max, col_tiles);
  if (KS > kMaxSplit) return hipErrorInvalidValue;
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes);
  hipLaunchKernelGGL(axpy_keyed_kernel, dim3(col_tiles, KS), dim3(1024), 0, s, a, keys, key_type,
                     thr, KS, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(partials, KS, 1, 1, a.d, a.alpha, a.out, a.d, a.accumulate, s);
}

}  // namespace sffn
