// SpAx three-tier read (abstract, Fig 2, Fig 3, Fig 4) and its offline
// encoder.
//
// Product: y = sum_{j in top} W^T[j] x_j + sum_{j in mid} What^T[j] x_j, with
// What^T[j][o] = zero_js + scale_js q_jo.  W^T rows (input columns j) are
// contiguous; a middle-tier column is one record: a 16-byte header of
// (fp16 scale, fp16 zero) per output segment, then 4-bit codes (output 2i in
// the low nibble of byte i).  The Q/K/V columns of one input are one record
// (Fig 4), so a selected column is one contiguous read in either tier.
//
// The grid is (512-column tiles) x (KS_top + KS_mid chunks): a workgroup
// streams either top rows (16-byte bf16 loads, 8 outputs per lane, four rows
// in flight) or middle rows (4-byte code loads, 8 outputs per lane, so both
// tiers share the lane -> output mapping; eight rows in flight, nine for
// keyed tiers).  The middle tier is decoded in registers:
// x_j * What[j][o] = (x_j scale_js) q_jo + x_j zero_js, where the second term
// is the same for all outputs of the segment and is summed once per lane.
// The tiers come as index lists (a chunk is a range of list items) or as two
// threshold pairs over the keys (a chunk is a range of inputs; the workgroup
// lists its tier's members in LDS first).  Partials are summed in chunk
// order by the shared split-K reduction.
#include <algorithm>

#include <hip/hip_fp16.h>

#include "sffn_splitk.h"

namespace sffn {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)h));
}

struct SegBounds { int b[5]; };

// Rows of one tier for this wave (items k0 + w + kWaves * u, u < nu): one
// vector load per lane fetches a row index (lane l: item u = ub + l), and
// the weight loads of a batch are then issued back to back from
// readlane-broadcast rows, with no branch around a load (padding slots of a
// batch re-read the wave's first row with x = 0).
template <int U, typename Issue, typename Accum>
__device__ __forceinline__ void tier_rows(const int32_t* idx, const float* x, int k0, int nu,
                                          Issue issue, Accum accum) {
  const int lane = threadIdx.x & 63, w = wave_id();
  for (int ub = 0; ub < nu; ub += 64) {
    const bool ok = ub + lane < nu;
    const int r = idx[k0 + w + kWaves * (ok ? ub + lane : 0)];
    const int nb = min(64, nu - ub);
    auto row_at = [&](int u) { return __builtin_amdgcn_readlane(r, u < nb ? u : 0); };
    for (int u = 0; u < nb; u += U) {
      issue(u, row_at);
      // gathered after the batch's weights were requested (r is a valid row
      // for every lane), so its wait is the batch's wait; the compiler
      // barrier keeps it here rather than hoisted ahead of the weights
      asm volatile("" ::: "memory");
      const float xr = x[r];
      const float xv = ok ? xr : 0.f;
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const float xu = u + uu < nb
            ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(xv), u + uu)) : 0.f;
        accum(uu, xu);
      }
    }
  }
}

// Keyed tiers: the workgroup forms its chunk's row list in LDS from the
// keys.  A tier's chunk m covers the inputs [m c, (m + 1) c), c <= 4096, in
// passes of 1024 (wave w tests the w-th 64 of a pass, one input per lane);
// input j is in the top tier iff it is in the set of thr_top, in the middle
// tier iff it is in the set of thr and not in the top tier (a pair (T, I)
// holds j iff key_j > T, or key_j == T and j <= I).  The members go to
// list[] in index order, and the waves then take its items round-robin as
// from a global list, so the rows are spread evenly over the waves.
// Returns the chunk's row count; every thread of the workgroup calls it.
constexpr int kKeyedPass = kWaves * 64;
constexpr int kKeyedPasses = 4;
constexpr int kKeyedChunk = kKeyedPass * kKeyedPasses;

__device__ __forceinline__ bool in_pair(uint32_t k, int j, uint32_t T, int I) {
  return k > T || (k == T && j <= I);
}

__device__ __forceinline__ uint32_t tier_key(const void* keys, int key_type, int j) {
  const uint32_t b = reinterpret_cast<const uint32_t*>(keys)[j];
  if (key_type == 0) return b & 0x7FFFFFFFu;
  if (key_type == 1) return b;
  return key_signed(__uint_as_float(b));
}

__device__ __forceinline__ int keyed_tier_list(const TierArgs& a, bool top, int m, int KS_t,
                                               int32_t* list, int* wcnt) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int c = (a.n_in + KS_t - 1) / KS_t;
  const int n0 = m * c, n1 = min(a.n_in, n0 + c);
  // every pass's keys requested up front (clamped reads past the chunk)
  uint32_t kv[kKeyedPasses];
#pragma unroll
  for (int p = 0; p < kKeyedPasses; ++p)
    kv[p] = tier_key(a.keys, a.key_type, min(n0 + p * kKeyedPass + w * 64 + lane, a.n_in - 1));
  const uint32_t Tt = a.thr_top[0], T = a.thr[0];
  const int It = (int)a.thr_top[1], I = (int)a.thr[1];
  int tot = 0;
#pragma unroll
  for (int p = 0; p < kKeyedPasses; ++p) {
    if (n0 + p * kKeyedPass >= n1) break;   // uniform
    const int j = n0 + p * kKeyedPass + w * 64 + lane;
    const bool it = in_pair(kv[p], j, Tt, It);
    const bool in = j < n1 && (top ? it : (in_pair(kv[p], j, T, I) && !it));
    const uint64_t mm = __ballot(in);
    if (lane == 0) wcnt[w] = (int)__popcll(mm);
    __syncthreads();
    int off = tot, pt = 0;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const int cv = wcnt[v];
      off += v < w ? cv : 0;
      pt += cv;
    }
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mm >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((uint32_t)mm, 0u));
    if (in) list[off + rank] = j;
    tot += pt;
    __syncthreads();   // the list is complete, and wcnt free for the next pass
  }
  return tot;
}

// UM: middle-tier rows in flight per lane (8 for index lists; 9 for keyed
// tiers, whose per-chunk row counts vary by about +-10% around the mean: at
// the 14336-input down projection nine keep the fullest chunks at two
// batches per wave).
template <int UM>
__global__ __launch_bounds__(1024) void tiered_kernel(TierArgs a, int KS_top, int KS_mid,
                                                      int xcd_order, float* partials) {
  __shared__ float4 red[kWaves][kTileCols / 4];
  __shared__ int32_t klist[kKeyedChunk];   // keyed tiers: the chunk's rows
  __shared__ int kcnt[kWaves];
  const int lane = threadIdx.x & 63, w = wave_id();
  int tile = blockIdx.x, ks = blockIdx.y;
  if (xcd_order) {
    // Workgroups go to the eight XCDs round-robin by linear id; remap so that
    // the column tiles of a row chunk run on one XCD (or two), and a chunk's
    // record headers and boundary lines are fetched into one L2.
    const int T = (int)gridDim.x, G = T * (int)gridDim.y;
    const int L = blockIdx.x + T * blockIdx.y;
    const int x = L & 7, sl = L >> 3;
    if (xcd_order == 1) {
      // chunk count a multiple of 8: XCD x takes chunks x, x + 8, ...
      tile = sl % T;
      ks = (sl / T) * 8 + x;
    } else {
      // otherwise XCD x takes a contiguous run of the (chunk, tile) sequence
      const int q = x * (G >> 3) + min(x, G & 7) + sl;
      tile = q % T;
      ks = q / T;
    }
  }
  const int col = tile * kTileCols + 8 * lane;
  const int colc = col < a.d_out ? col : 0;   // lanes past the last output re-read output 0

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  if (ks < KS_top) {
    constexpr int U = 4;
    uint4 wv[U];
    auto issue = [&](int u, auto row_at) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu)
        wv[uu] = load_stream16(a.Wt + (size_t)row_at(u + uu) * a.ld_w + colc);
    };
    auto accum = [&](int uu, float xu) {
      float f[8];
      unpack8(wv[uu], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(xu, f[e], acc[e]);
    };
    if (a.thr) {
      const int n = keyed_tier_list(a, true, ks, KS_top, klist, kcnt);
      const int nu = n > w ? (n - w + kWaves - 1) / kWaves : 0;
      tier_rows<U>(klist, a.x, 0, nu, issue, accum);
    } else {
      int n = a.cnt_top ? *a.cnt_top : 0;
      n = n < a.k_top_max ? n : a.k_top_max;
      n = n > 0 ? n : 0;
      const int chunk = (n + KS_top - 1) / KS_top;
      const int k0 = ks * chunk, k1 = min(n, k0 + chunk);
      const int nu = k1 - k0 > w ? (k1 - k0 - w + kWaves - 1) / kWaves : 0;
      tier_rows<U>(a.idx_top, a.x, k0, nu, issue, accum);
    }
  } else {
    const int m = ks - KS_top;
    int seg = 0;
#pragma unroll
    for (int s = 1; s < 4; ++s)
      if (s < a.n_seg && colc >= a.seg_bounds[s]) seg = s;
    const int hdr_off = 4 * seg;
    const int code_off = 16 + (colc >> 1);
    float zacc = 0.f;
    constexpr int U = UM;
    uint32_t hdr[U], codes[U];
    auto issue = [&](int u, auto row_at) {
#pragma unroll
      for (int uu = 0; uu < U; ++uu) {
        const uint8_t* rec = a.rec + (size_t)row_at(u + uu) * a.rec_bytes;
        hdr[uu] = *reinterpret_cast<const uint32_t*>(rec + hdr_off);
        codes[uu] = load_stream4(rec + code_off);
      }
    };
    auto accum = [&](int uu, float xu) {
      const float sc = half_bits_to_float(hdr[uu] & 0xFFFFu);
      const float z = half_bits_to_float(hdr[uu] >> 16);
      const float sx = xu * sc;
      zacc = fmaf(xu, z, zacc);
      const uint32_t lo = codes[uu] & 0x0F0F0F0Fu;
      const uint32_t hi = (codes[uu] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        acc[2 * b] = fmaf(sx, (float)((lo >> (8 * b)) & 0xFFu), acc[2 * b]);
        acc[2 * b + 1] = fmaf(sx, (float)((hi >> (8 * b)) & 0xFFu), acc[2 * b + 1]);
      }
    };
    if (a.thr) {
      const int n = keyed_tier_list(a, false, m, KS_mid, klist, kcnt);
      const int nu = n > w ? (n - w + kWaves - 1) / kWaves : 0;
      tier_rows<U>(klist, a.x, 0, nu, issue, accum);
    } else {
      int n = a.cnt_mid ? *a.cnt_mid : 0;
      n = n < a.k_mid_max ? n : a.k_mid_max;
      n = n > 0 ? n : 0;
      const int chunk = (n + KS_mid - 1) / KS_mid;
      const int k0 = m * chunk, k1 = min(n, k0 + chunk);
      const int nu = k1 - k0 > w ? (k1 - k0 - w + kWaves - 1) / kWaves : 0;
      tier_rows<U>(a.idx_mid, a.x, k0, nu, issue, accum);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += zacc;
  }

  const float part = wg_reduce_cols(red, acc);
  const int c = tile * kTileCols + (int)threadIdx.x;
  if (threadIdx.x < kTileCols && c < a.d_out) partials[(size_t)ks * a.d_out + c] = part;
}

int tiered_keyed_min_chunks(int n_in) { return (n_in + kKeyedChunk - 1) / kKeyedChunk; }

hipError_t launch_tiered(const TierArgs& a, hipStream_t s) {
  const int col_tiles = (a.d_out + kTileCols - 1) / kTileCols;
  // One round of workgroups, one per CU (a second partial round costs more
  // than it adds).  The chunk slots are split between the tiers by row
  // count, top rows weighted 1.3 (1.45 for keyed tiers, with nine middle
  // rows in flight): measured on MI355X, a middle-tier row (4-bit codes
  // decoded in registers) takes about as long as a top-tier row although it
  // is a quarter of the bytes.  A chunk keeps at least one row per wave.
  const long slots = std::max(1, 256 / col_tiles);
  const long kt = std::max(0, a.k_top_max), km = std::max(0, a.k_mid_max);
  long ks_top = 0, ks_mid = 0;
  if (kt + km > 0) {
    const double wt = (a.thr ? 1.45 : 1.3) * (double)kt, wm = (double)km;
    ks_top = kt > 0 ? std::max(1L, (long)(slots * wt / (wt + wm) + 0.5)) : 0;
    if (km > 0 && ks_top >= slots) ks_top = std::max(1L, slots - 1);
    ks_mid = km > 0 ? std::max(1L, slots - ks_top) : 0;
    ks_top = std::min(ks_top, (kt + kWaves - 1) / kWaves);
    ks_mid = std::min(ks_mid, (km + kWaves - 1) / kWaves);
  }
  if (a.thr) {
    // keyed tiers: the sizes are hints only (the pairs decide the tiers), so
    // each tier's chunks cover all inputs, at most 4096 per chunk
    // (raised, one tier is then given back slots from the other where it can)
    const long need = tiered_keyed_min_chunks(a.n_in);
    ks_top = std::max(ks_top, need);
    ks_mid = std::max(ks_mid, need);
    if (ks_top + ks_mid > slots) ks_top = std::max(need, std::min(ks_top, slots - ks_mid));
    if (ks_top + ks_mid > slots) ks_mid = std::max(need, slots - ks_top);
  }
  ks_top = std::min<long>(ks_top, kMaxSplit / 2);
  ks_mid = std::min<long>(ks_mid, kMaxSplit / 2);
  if (ks_top + ks_mid == 0) ks_mid = 1;   // nothing to read: one chunk writes y
  // XCD-grouped block order where the chunk count allows it (measured on the
  // 14336 -> 4096 down projection: 13.0 -> 11.9 us; with 12 column tiles and
  // 21 chunks the plain order is kept)
  const int xcd_order = (ks_top + ks_mid) % 8 == 0 ? 1 : 2;
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes);
  if (a.thr)
    hipLaunchKernelGGL(tiered_kernel<9>, dim3(col_tiles, (unsigned)(ks_top + ks_mid)), dim3(1024), 0,
                       s, a, (int)ks_top, (int)ks_mid, xcd_order, partials);
  else
    hipLaunchKernelGGL(tiered_kernel<8>, dim3(col_tiles, (unsigned)(ks_top + ks_mid)), dim3(1024), 0,
                       s, a, (int)ks_top, (int)ks_mid, xcd_order, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(partials, (int)(ks_top + ks_mid), 1, 1, a.d_out, nullptr, a.y,
                              a.d_out, a.accumulate, s);
}

// ------------------------------------------------------------------ encoder

__global__ __launch_bounds__(256) void encode_kernel(const uint16_t* __restrict__ Wt, int ld_w,
                                                     int n_in, SegBounds sb, int n_seg,
                                                     uint8_t* __restrict__ rec, int rec_bytes) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + wave_id();
  const int j = gw / n_seg, s = gw - (gw / n_seg) * n_seg;
  if (j >= n_in) return;
  const int lo = sb.b[s], hi = sb.b[s + 1];
  const int nch = (hi - lo) >> 3;
  const uint16_t* wr = Wt + (size_t)j * ld_w + lo;

  float mn = __uint_as_float(0x7F800000u), mx = -mn;
  for (int c = lane; c < nch; c += 64) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(wr + 8 * c), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) { mn = fminf(mn, f[e]); mx = fmaxf(mx, f[e]); }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  }
  const __half zh = __float2half_rn(mn);
  const float z32 = __half2float(zh);
  const __half sh = __float2half_rn(__fdiv_rn(mx - z32, 15.0f));
  const float s32 = __half2float(sh);

  uint8_t* r = rec + (size_t)j * rec_bytes;
  for (int c = lane; c < nch; c += 64) {
    float f[8];
    unpack8(*reinterpret_cast<const uint4*>(wr + 8 * c), f);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float q = 0.f;
      if (s32 != 0.f) q = fminf(fmaxf(rintf(__fdiv_rn(f[e] - z32, s32)), 0.f), 15.f);
      word |= ((uint32_t)q) << (4 * e);   // output lo+8c+e: byte e/2, low nibble if e even
    }
    *reinterpret_cast<uint32_t*>(r + 16 + ((lo + 8 * c) >> 1)) = word;
  }
  if (lane == 0) {
    *reinterpret_cast<uint32_t*>(r + 4 * s) =
        (uint32_t)__half_as_ushort(sh) | ((uint32_t)__half_as_ushort(zh) << 16);
    if (s == 0)
      for (int u = n_seg; u < 4; ++u) *reinterpret_cast<uint32_t*>(r + 4 * u) = 0u;
  }
}

hipError_t launch_encode_tiers(const uint16_t* Wt, int ld_w, int n_in, int d_out,
                               const int* seg_bounds, int n_seg, uint8_t* rec, int rec_bytes,
                               hipStream_t s) {
  (void)d_out;
  SegBounds sb{};
  for (int i = 0; i <= n_seg; ++i) sb.b[i] = seg_bounds[i];
  const long waves = (long)n_in * n_seg;
  hipLaunchKernelGGL(encode_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, Wt, ld_w,
                     n_in, sb, n_seg, rec, rec_bytes);
  return hipGetLastError();
}

}  // namespace sffn
