// Activations for several tokens at once on MFMA (batched decode, and the
// dense prefill / calibration passes that feed the selection).
//
// C[m][n] = sum_k X[m][k] W[n][k]: tokens are the M dimension, neurons the
// N dimension.  The fp32 activations are split into bf16 hi + lo parts
// (x = hi + lo to ~2^-17 relative) and contracted with two MFMAs into one
// fp32 accumulator, so the result keeps fp32-grade accuracy with bf16
// weights.
//
// Work split: a workgroup owns two 16-neuron x 16-token tiles; two waves
// share a tile, one per half of K, and their accumulators are added in LDS
// at the end (so a CU keeps twice the loads in flight that one wave per tile
// would).  K is walked in chunks of 128: a wave loads its 16 rows (per
// weight matrix) with row-contiguous 16-byte loads (four rows of 256 bytes
// per instruction, not 16 rows of 64 bytes as the MFMA operand layout would
// read them), stores them in its own LDS area, and reads them back in the
// B-operand layout (lane (n, g) takes 8 consecutive k of row n).  The next
// chunk's weights and activations are in flight while the current chunk is
// contracted.
//
// Packed weights (row tiles, see sffn_device.h): the same work split and
// arithmetic; only the addresses differ, so results are bitwise those of the
// row-major layout.
//
// Balance (dense row ops with a workspace): a layer whose tile pairs do not
// split evenly over the 256 CUs (17408 neurons = 544 pairs: a third of the
// CUs would carry a third workgroup) runs the largest multiple of 256 pairs
// as above and splits the remaining pairs along K into Q slices (about
// kSliceBudget short workgroups in all).  A slice writes its accumulators and its
// part of each token's sum of squares to the workspace; a fix-up kernel adds
// the Q slices in slice order and applies the same epilogue.
#include <algorithm>

#include "sffn_device.h"

namespace sffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // register / LDS vector

enum { kOpGlu = 0, kOpDotRelu = 1, kOpGated = 2, kOpDot = 4 };

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Split 8 fp32 values into bf16 hi and lo parts (packed pairs, memory order).
__device__ __forceinline__ uint32_t split_pair(float v0, float v1, uint32_t& lo) {
  const uint32_t h0 = f32_to_bf16_rne(v0), h1 = f32_to_bf16_rne(v1);
  const uint32_t l0 = f32_to_bf16_rne(v0 - __uint_as_float(h0 << 16));
  const uint32_t l1 = f32_to_bf16_rne(v1 - __uint_as_float(h1 << 16));
  lo = l0 | (l1 << 16);
  return h0 | (h1 << 16);
}

__device__ __forceinline__ void split8(const float4& p, const float4& q, uint4& hi, uint4& lo) {
  hi.x = split_pair(p.x, p.y, lo.x);
  hi.y = split_pair(p.z, p.w, lo.y);
  hi.z = split_pair(q.x, q.y, lo.z);
  hi.w = split_pair(q.z, q.w, lo.w);
}

constexpr int kKC = 128;                    // k per chunk
constexpr int kRowU4 = kKC / 8;             // 16-byte groups of bf16 per chunk row
constexpr int kPitch = kRowU4 + 1;          // LDS row pitch: rows start 4 banks apart

// Epilogue of one lane: tokens m0 + 4g + i (i < 4) of neuron row my_row, from
// the full-K accumulators and the tokens' sums of squares.
template <int OP>
__device__ __forceinline__ void mfma_epilogue(const RowOpArgs& a, const f32x4& acc0,
                                              const f32x4& acc1, const float* sq_tok, int m0,
                                              int g, int my_row) {
  // C layout of the 16x16 MFMA: lane l, register i holds row m = 4*(l/16)+i
  // (token) and column n = l%16 (neuron).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    const int b = m0 + m;
    if (b >= a.batch) continue;
    const float ss = sq_tok[m];
    // optional unit-gain RMSNorm of token b's input, applied to the dot products
    const float inv = a.rms_eps > 0.f ? 1.f / sqrtf(ss / (float)a.d + a.rms_eps) : 1.f;
    float v;
    if (OP == kOpGlu) {
      const float gg = acc0[i] * inv;
      v = (gg / (1.f + expf(-gg))) * (acc1[i] * inv);
    } else if (OP == kOpDotRelu) {
      v = fmaxf(acc0[i] * inv - a.tau_scale * sqrtf(ss) * inv, 0.f);
    } else if (OP == kOpGated) {
      v = a.aux[(size_t)b * a.ld_aux + my_row] * (acc1[i] * inv);
    } else {
      v = acc0[i] * inv;
    }
    if (a.accumulate) v += a.out[(size_t)b * a.ld_out + my_row];
    a.out[(size_t)b * a.ld_out + my_row] = v;
    if (a.key_out) a.key_out[(size_t)b * a.ld_out + my_row] = key_abs(v);
  }
}

// Workspace record of one K slice of one tile and token tile: acc0 and acc1
// as [lane][4] (the MFMA C layout) and the 16 tokens' partial sums of squares.
constexpr int kSliceFloats = 2 * 256 + 16;

// blockIdx.x < G_main: a pair of 16-neuron tiles over all of K.  Otherwise
// slice q of the pair G_main + (blockIdx.x - G_main) / Q, over K chunks
// [q nch / Q, (q + 1) nch / Q), its accumulators written to slices.
template <int OP>
__global__ __launch_bounds__(256) void rowop_mfma_kernel(RowOpArgs a, int G_main, int Q,
                                                         float* slices) {
  constexpr bool kW0 = OP != kOpGated;
  constexpr bool kW1 = OP == kOpGlu || OP == kOpGated;
  constexpr int kMat = (kW0 && kW1) ? 2 : 1;
  __shared__ u32x4 stage[4][kMat][16][kPitch];   // each wave's 16 weight rows of its chunk
  __shared__ u32x4 xs[2][2][16][kPitch];         // [half][hi / lo][token][k group]
  __shared__ float sq_tok[16];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = wave_id();
  const int tile = w >> 1, half = w & 1;       // two 16-neuron tiles x two halves of K
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int m0 = blockIdx.y * 16;
  const bool sliced = (int)blockIdx.x >= G_main;
  const int pair = sliced ? G_main + ((int)blockIdx.x - G_main) / Q : (int)blockIdx.x;
  const int slice = sliced ? ((int)blockIdx.x - G_main) % Q : 0;
  const int t0 = (pair * 2 + tile) * 16;   // this wave's first item

  int n_items;
  if (a.idx) {
    int c = *a.count;
    c = c < a.k_max ? c : a.k_max;
    n_items = (c > 0 ? c : 0) * a.group;
  } else {
    n_items = a.n_rows;
  }
  // A workgroup with no live item has nothing to do (uniform exit, before
  // any barrier).  Otherwise items past the end re-read the last live item's
  // row (a selected row: skipped rows are never read) and tokens past the
  // batch read token 0: an MFMA output (m, n) depends only on A row m and
  // B column n, so those lanes only produce outputs that are never stored.
  if (pair * 32 >= n_items) return;
  auto item_to_row = [&](int it) -> int {
    it = it < n_items ? it : n_items - 1;
    if (!a.idx) return it;
    const int q = it / a.group;
    return a.idx[q] * a.group + (it - q * a.group);
  };
  // weight loader: lane l loads rows 4i + (l >> 4), 16 bytes at k-offset
  // 8*(l & 15).  Row-major: row r at r * ld_w, chunk c at 128 c.  Packed row
  // tiles: the 16 rows of a tile and the 128 k of a chunk are one contiguous
  // 4 KB block (a wave's chunk is one sequential read), chunk c 16 * 128 c on.
  const size_t kstep = a.packed ? 16 : 1;
  size_t woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = item_to_row(t0 + 4 * i + (lane >> 4));
    woff[i] = a.packed ? (size_t)(r >> 4) * 16 * a.d + (size_t)(r & 15) * kKC + 8 * (lane & 15)
                       : (size_t)r * a.ld_w + 8 * (lane & 15);
  }
  const int my_row = item_to_row(t0 + nl);          // output column of this lane
  const bool my_live = t0 + nl < n_items;
  // activation loader: thread t loads token t >> 4, k-offset 8*(t & 15) of
  // both halves' chunks
  const int xt = t >> 4, xg = t & 15;
  const int xtok = m0 + xt < a.batch ? m0 + xt : 0;
  const float* xsrc = a.x + (size_t)xtok * a.ld_in + 8 * xg;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float sq = 0.f;        // this thread's share of token xt's sum of squares (chunks)
  float sq_tail = 0.f;   // token nl's squares in k-group g of the tail

  // chunks of 128 k: this workgroup's range [cb, ce) (all of K, or a slice);
  // the first half of it takes [cb, cb + nA), the second the rest
  const int nch = a.d / kKC;
  const int cb = sliced ? slice * nch / Q : 0;
  const int ce = sliced ? (slice + 1) * nch / Q : nch;
  const int nA = (ce - cb + 1) / 2, nB = ce - cb - nA;
  const int my_n = half ? nB : nA;
  const int my_c0 = cb + (half ? nA : 0);
  // the k past the last chunk (row-major only: packed rows have d % 128 == 0)
  const bool has_tail = ce == nch && nch * kKC < a.d && !a.packed;
  u32x4 wr0[4], wr1[4];   // in-flight weights (this lane's share of its next chunk)
  float4 xr[2][2];        // in-flight activations: [half][8 values]
  auto load_chunk = [&](int c) {
    if (c < my_n) {
      const int k = (my_c0 + c) * kKC;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kW0) wr0[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.W0 + woff[i] + k * kstep));
        if (kW1) wr1[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.W1 + woff[i] + k * kstep));
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (c < (h ? nB : nA)) {
        const int k = (cb + (h ? nA : 0) + c) * kKC;
        xr[h][0] = *reinterpret_cast<const float4*>(xsrc + k);
        xr[h][1] = *reinterpret_cast<const float4*>(xsrc + k + 4);
      }
    }
  };
  if (nA > 0) load_chunk(0);
  for (int c = 0; c < nA; ++c) {
    __syncthreads();              // the previous chunk's LDS reads are done
    {
      const int rr = lane >> 4, cc = lane & 15;
      if (c < my_n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (kW0) stage[w][0][4 * i + rr][cc] = wr0[i];
          if (kW1) stage[w][kMat - 1][4 * i + rr][cc] = wr1[i];
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (c < (h ? nB : nA)) {
          const float4 p = xr[h][0], q = xr[h][1];
          sq = fmaf(p.x, p.x, sq); sq = fmaf(p.y, p.y, sq);
          sq = fmaf(p.z, p.z, sq); sq = fmaf(p.w, p.w, sq);
          sq = fmaf(q.x, q.x, sq); sq = fmaf(q.y, q.y, sq);
          sq = fmaf(q.z, q.z, sq); sq = fmaf(q.w, q.w, sq);
          uint4 hh, ll;
          split8(p, q, hh, ll);
          xs[h][0][xt][xg] = (u32x4){hh.x, hh.y, hh.z, hh.w};
          xs[h][1][xt][xg] = (u32x4){ll.x, ll.y, ll.z, ll.w};
        }
      }
    }
    __syncthreads();
    if (c + 1 < nA) load_chunk(c + 1);
    if (c < my_n) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        // A operand: token nl, k = 32 s + 8 g; B operand: row nl, same k
        const u32x4 ah = xs[half][0][nl][4 * s + g], al = xs[half][1][nl][4 * s + g];
        if (kW0) {
          const u32x4 b = stage[w][0][nl][4 * s + g];
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah), __builtin_bit_cast(bf16x8, b), acc0, 0, 0, 0);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al), __builtin_bit_cast(bf16x8, b), acc0, 0, 0, 0);
        }
        if (kW1) {
          const u32x4 b = stage[w][kMat - 1][nl][4 * s + g];
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah), __builtin_bit_cast(bf16x8, b), acc1, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al), __builtin_bit_cast(bf16x8, b), acc1, 0, 0, 0);
        }
      }
    }
  }
  // tail (d not a multiple of 128), taken by the second-half waves of the
  // workgroup holding the last chunk: one 32-k step at a time, straight
  // from memory
  if (half == 1 && has_tail) {
    for (int k = nch * kKC; k < a.d; k += 32) {
      const float* xp = a.x + (size_t)(m0 + nl < a.batch ? m0 + nl : 0) * a.ld_in + k + 8 * g;
      const float4 p = *reinterpret_cast<const float4*>(xp);
      const float4 q = *reinterpret_cast<const float4*>(xp + 4);
      // lane (nl, g) holds token nl's k-group g (the same in both such waves; wave 1's count is used)
      sq_tail = fmaf(p.x, p.x, sq_tail); sq_tail = fmaf(p.y, p.y, sq_tail);
      sq_tail = fmaf(p.z, p.z, sq_tail); sq_tail = fmaf(p.w, p.w, sq_tail);
      sq_tail = fmaf(q.x, q.x, sq_tail); sq_tail = fmaf(q.y, q.y, sq_tail);
      sq_tail = fmaf(q.z, q.z, sq_tail); sq_tail = fmaf(q.w, q.w, sq_tail);
      uint4 xh, xl;
      split8(p, q, xh, xl);
      const size_t off = (size_t)my_row * a.ld_w + k + 8 * g;
      if (kW0) {
        const uint4 b = *reinterpret_cast<const uint4*>(a.W0 + off);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xh), as_bf16x8(b), acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xl), as_bf16x8(b), acc0, 0, 0, 0);
      }
      if (kW1) {
        const uint4 b = *reinterpret_cast<const uint4*>(a.W1 + off);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xh), as_bf16x8(b), acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xl), as_bf16x8(b), acc1, 0, 0, 0);
      }
    }
  }

  // token sums of squares: the chunk part is spread over the 16 loader threads
  // of each token (lanes 16j..16j+15 of a wave); the tail part over the four
  // k-groups of wave 1's lanes nl + 16 g.  Both are combined through LDS in a
  // fixed order, and the second halves' accumulators are handed to the first
  // halves.
  {
    float v = sq;
    v += __shfl_xor(v, 1, kWave); v += __shfl_xor(v, 2, kWave);
    v += __shfl_xor(v, 4, kWave); v += __shfl_xor(v, 8, kWave);
    float tv = sq_tail;
    tv += __shfl_xor(tv, 16, kWave); tv += __shfl_xor(tv, 32, kWave);
    __syncthreads();   // every wave is past its last chunk: the staging area is free
    // the second halves' accumulators, [tile][matrix][lane], in the staging area
    f32x4(*comb)[kMat][64] = reinterpret_cast<f32x4(*)[kMat][64]>(&stage[0][0][0][0]);
    if (xg == 0) sq_tok[xt] = v;
    if (half == 1) {
      if (kW0) comb[tile][0][lane] = acc0;
      if (kW1) comb[tile][kMat - 1][lane] = acc1;
    }
    __syncthreads();
    if (t >= 64 && t < 80 && has_tail) sq_tok[t - 64] += tv;
    __syncthreads();
  }
  if (half == 1) return;
  {
    const f32x4(*comb)[kMat][64] = reinterpret_cast<const f32x4(*)[kMat][64]>(&stage[0][0][0][0]);
    if (kW0) acc0 += comb[tile][0][lane];
    if (kW1) acc1 += comb[tile][kMat - 1][lane];
  }
  if (sliced) {
    // this slice's record of the tile: tiles are numbered from the first
    // sliced pair, records [tile][token tile][slice]
    const int st = (pair - G_main) * 2 + tile;
    float* rec = slices + ((size_t)(st * (int)gridDim.y + (int)blockIdx.y) * Q + slice) * kSliceFloats;
    *reinterpret_cast<f32x4*>(rec + 4 * lane) = acc0;
    *reinterpret_cast<f32x4*>(rec + 256 + 4 * lane) = acc1;
    if (lane < 16) rec[512 + lane] = sq_tok[lane];
    return;
  }
  if (!my_live) return;
  mfma_epilogue<OP>(a, acc0, acc1, sq_tok, m0, g, my_row);
}

// Fix-up of the sliced tiles: one wave per (tile, token tile) adds the Q
// slice records in slice order and applies the epilogue.
template <int OP>
__global__ __launch_bounds__(64) void rowop_mfma_fixup(RowOpArgs a, int first_tile, int Q,
                                                       const float* __restrict__ slices) {
  __shared__ float sq_tok[16];
  const int lane = threadIdx.x;
  const int st = blockIdx.x;
  const int t0 = (first_tile + st) * 16;
  const int n_items = a.n_rows;   // dense row ops only
  if (t0 >= n_items) return;
  const int nl = lane & 15, g = lane >> 4;
  const float* rec = slices + (size_t)(st * (int)gridDim.y + (int)blockIdx.y) * Q * kSliceFloats;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float ss = 0.f;
  for (int q = 0; q < Q; ++q) {
    const float* r = rec + (size_t)q * kSliceFloats;
    acc0 += *reinterpret_cast<const f32x4*>(r + 4 * lane);
    acc1 += *reinterpret_cast<const f32x4*>(r + 256 + 4 * lane);
    if (lane < 16) ss += r[512 + lane];
  }
  if (lane < 16) sq_tok[lane] = ss;
  __syncthreads();
  const int it = t0 + nl;
  if (it >= n_items) return;
  mfma_epilogue<OP>(a, acc0, acc1, sq_tok, (int)blockIdx.y * 16, g, it);
}

// Sliced workgroups per token tile: 128 (half a short workgroup per CU)
// measured 1-4% faster than 256 or 512 on the 17408 x 5120 layer at batch 8
// and 16 (gate/up 84 -> 74 us at batch 16 against the unsplit launch).
constexpr long kSliceBudget = 128;

template <int OP>
static hipError_t launch_op(const RowOpArgs& a, dim3 grid, int G_main, int Q, int first_tile,
                            int n_slice_tiles, float* slices, hipStream_t s) {
  hipLaunchKernelGGL(rowop_mfma_kernel<OP>, grid, dim3(256), 0, s, a, G_main, Q, slices);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_slice_tiles == 0) return e;
  hipLaunchKernelGGL(rowop_mfma_fixup<OP>, dim3(n_slice_tiles, grid.y), dim3(64), 0, s, a,
                     first_tile, Q, slices);
  return hipGetLastError();
}

hipError_t launch_rowop_mfma(const RowOpArgs& a, hipStream_t s) {
  const long items = a.idx ? (long)a.k_max * a.group : (long)a.n_rows;
  const int mt = (a.batch + 15) / 16;
  if (items == 0) return hipSuccess;
  // 2 tiles of 16 neurons x 2 halves of K per workgroup
  const long pairs = (items + 31) / 32;
  long G_main = pairs, Q = 1, sliced_pairs = 0;
  const int nch = a.d / kKC;
  if (!a.idx && a.ws && nch >= 2 && pairs >= 256 && pairs % 256 != 0) {
    // the largest multiple of 256 pairs over all of K; the rest in K slices
    const long r = pairs % 256;
    const long q = std::min<long>(std::max<long>(kSliceBudget / r, 1), nch);
    const size_t need = kWsHeaderBytes + (size_t)(2 * r) * mt * q * kSliceFloats * sizeof(float);
    if (q >= 2 && need <= a.ws_bytes) {
      G_main = pairs - r;
      Q = q;
      sliced_pairs = r;
    }
  }
  float* slices = sliced_pairs
      ? reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes) : nullptr;
  const int first_tile = (int)(2 * G_main);
  const int n_slice_tiles = (int)std::min<long>(2 * sliced_pairs, (items + 15) / 16 - first_tile);
  dim3 grid((unsigned)(G_main + sliced_pairs * Q), mt);
  switch (a.op) {
    case kOpGlu: return launch_op<kOpGlu>(a, grid, (int)G_main, (int)Q, first_tile,
                                          sliced_pairs ? n_slice_tiles : 0, slices, s);
    case kOpDotRelu: return launch_op<kOpDotRelu>(a, grid, (int)G_main, (int)Q, first_tile,
                                                  sliced_pairs ? n_slice_tiles : 0, slices, s);
    case kOpGated: return launch_op<kOpGated>(a, grid, (int)G_main, (int)Q, first_tile,
                                              sliced_pairs ? n_slice_tiles : 0, slices, s);
    default: return launch_op<kOpDot>(a, grid, (int)G_main, (int)Q, first_tile,
                                      sliced_pairs ? n_slice_tiles : 0, slices, s);
  }
}

}  // namespace sffn
