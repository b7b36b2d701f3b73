// Rank-range selection and compaction (one workgroup per row).
//
// The entries of a row are ordered by (key descending, index ascending) and
// the ranks [r_lo, r_hi) are selected: per-token top-alpha, top-beta by
// frequency and the top-delta base set of SelectInfer (§4, §5) are ranges
// [0, k); the SpAx middle tier (Fig 2) is [k_top, k_top + k_mid), and the
// same call can also emit the ranks [0, r_lo) (the SpAx top tier) as a
// second list.  With cluster > 1 an entry is a block of `cluster` contiguous
// values whose key is the largest key of the block (PowerInfer-2 guide,
// "Neuron Cluster Decomposition": the cluster is the unit that is selected).
//
// Method: NT threads; thread t owns the entries j*NT + t (j < KPT), so every
// load and every mask store of a wave is contiguous.  One workgroup handles
// a row (at most 32768 entries), so the cost is the instructions each wave
// issues and the chain of barriers; the kernel keeps both short.
//  1. The largest eligible key (an OR over the row) fixes the most
//     significant bit that varies, so the digits start there: keys that fit
//     in 11 bits (e.g. frequency counts) take one pass, float magnitudes 3.
//  2. MSB-first radix search finds, for each bound r in {r_hi, r_lo}, the key
//     T_r of the r-th largest entry, how many entries equal to T_r fall
//     inside the top r, and how many equal T_r in all.  Both bounds share
//     one LDS histogram (16-bit halves of one counter); wave 0 scans it with
//     DPP lane moves.  After the first pass only the keys whose higher
//     digits match a bound can matter: each thread tests its own keys and
//     only those are counted in the later passes.  A bound that covers every
//     eligible entry needs no search (pure compaction, e.g. the nonzero
//     clusters of a ReLU layer).
//  3. Index-order positions come from wave ballots: an entry's position
//     among the entries with some property is the count in the (j, wave)
//     blocks before its own plus the count of lower lanes in its ballot.
//     This places the selected indices (ascending lists, contiguous stores)
//     and, when T_r is tied across the bound, ranks the tied entries in
//     index order, which decides them as the (key desc, index asc) order
//     does.
// Everything is integer: the result is unique and bit-exact.
#include "sffn_device.h"

namespace sffn {

constexpr int kMaxClusters = 4096;   // entries of a row in cluster mode

// Inclusive scan over the 64 lanes of a wave with DPP moves: shifts of 1, 2,
// 4, 8 within each row of 16 lanes, then rows 1 and 3 take lane 15 of the
// row below and rows 2 and 3 take lane 31.  Lanes a move leaves out get 0.
template <bool kOr>
__device__ __forceinline__ uint32_t wave_incl(uint32_t x) {
#define SFFN_DPP_STEP(ctrl, rows, bc)                                                      \
  {                                                                                        \
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, rows, 0xf, bc); \
    x = kOr ? (x | y) : (x + y);                                                           \
  }
  SFFN_DPP_STEP(0x111, 0xf, true)
  SFFN_DPP_STEP(0x112, 0xf, true)
  SFFN_DPP_STEP(0x114, 0xf, true)
  SFFN_DPP_STEP(0x118, 0xf, true)
  SFFN_DPP_STEP(0x142, 0xa, false)
  SFFN_DPP_STEP(0x143, 0xc, false)
#undef SFFN_DPP_STEP
  return x;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint32_t key_of_bits(int key_type, uint32_t b) {
  if (key_type == 0) return b & 0x7FFFFFFFu;
  if (key_type == 1) return b;
  return key_signed(__uint_as_float(b));
}

// Index-order positions of two per-entry predicates, given as bit masks
// (bit j: entry j*NT + t).  ordered_counts stores the packed (hi half, lo
// half) count of every (j, wave) block; after a barrier, ordered_offsets
// gives lane j the packed count of all blocks before (j, this wave) and the
// totals; an entry's position is then that offset (read from lane j) plus
// the number of lower lanes in its ballot.
template <int NT, int KPT, bool TWO>
__device__ __forceinline__ void ordered_counts(uint32_t bits_h, uint32_t bits_l,
                                               uint32_t (*cnt)[NT / 64]) {
  const int lane = threadIdx.x & 63, w = wave_id();
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t bh = __ballot((bits_h >> j) & 1u);
    const uint64_t bl = TWO ? __ballot((bits_l >> j) & 1u) : 0ull;
    if (lane == 0) cnt[j][w] = ((uint32_t)__popcll(bh) << 16) | (uint32_t)__popcll(bl);
  }
}

template <int NT, int KPT>
__device__ __forceinline__ uint32_t ordered_offsets(uint32_t (*cnt)[NT / 64], uint32_t& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, w = wave_id();
  uint32_t row_total = 0, row_below = 0;
  if (lane < KPT) {
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const uint32_t c = cnt[lane][ww];
      row_total += c;
      row_below += ww < w ? c : 0u;
    }
  }
  const uint32_t incl = wave_incl<false>(row_total);
  total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  return incl - row_total + row_below;
}

template <bool TWO>
__device__ __forceinline__ uint32_t ordered_pos(uint32_t off_j, uint32_t bits_h, uint32_t bits_l,
                                                int j) {
  const uint64_t bh = __ballot((bits_h >> j) & 1u);
  if (!TWO) return off_j + (lanes_below(bh) << 16);
  const uint64_t bl = __ballot((bits_l >> j) & 1u);
  return off_j + ((lanes_below(bh) << 16) | lanes_below(bl));
}

// Wave 0's scan of one radix pass over nb bins (nb <= 2048, H 16-byte
// aligned): for each bound it writes the digit holding rank `rem` (in the
// packed counters' hi or lo half), the rank left inside that digit and the
// digit's count.  Lane l holds q = nb/64 consecutive bins (lane 0 the
// largest digits), read as 16-byte vectors; a DPP scan gives the counts
// above each lane, and the lane that holds the rank walks its bins from the
// top.
__device__ __forceinline__ void scan_pass(const uint32_t* H, int nb, bool want_hi, uint32_t rem_hi,
                                          bool want_lo, uint32_t rem_lo, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  uint32_t h[32];
  int q, base;
  if (nb >= 256) {   // 4..32 bins per lane
    q = nb >> 6;
    base = nb - q * (lane + 1);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint4 v = 4 * c < q ? *reinterpret_cast<const uint4*>(H + base + 4 * c)
                                : make_uint4(0u, 0u, 0u, 0u);
      h[4 * c] = v.x; h[4 * c + 1] = v.y; h[4 * c + 2] = v.z; h[4 * c + 3] = v.w;
    }
  } else {           // at most 4 bins per lane: one bin per lane
    q = 1;
    base = nb - 1 - lane;
#pragma unroll
    for (int i = 0; i < 32; ++i) h[i] = 0u;
    h[0] = base >= 0 ? H[base] : 0u;
    if (nb > 64) {   // 128 bins: two per lane
      q = 2;
      base = nb - 2 * (lane + 1);
      h[0] = H[base];
      h[1] = H[base + 1];
    }
  }
  // group sums of 4 bins, then the lane total
  uint32_t g4[8];
  uint32_t own = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    g4[c] = h[4 * c] + h[4 * c + 1] + h[4 * c + 2] + h[4 * c + 3];
    own += g4[c];
  }
  const uint32_t above = wave_incl<false>(own) - own;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const bool want = b == 0 ? want_hi : want_lo;
    if (!want) continue;
    const int half = b == 0 ? 16 : 0;
    const uint32_t rem = b == 0 ? rem_hi : rem_lo;
    const uint32_t acc0 = (above >> half) & 0xFFFFu;
    if (!(acc0 < rem && rem <= acc0 + ((own >> half) & 0xFFFFu))) continue;   // one lane
    // the group of 4 bins holding the rank, then the bin (descending digits);
    // once the rank is passed, acc >= rem and no later group can match
    uint32_t acc = acc0, acc_at = acc0;
    int gsel = 0;
#pragma unroll
    for (int c = 7; c >= 0; --c) {
      const uint32_t n = (g4[c] >> half) & 0xFFFFu;
      if (acc < rem && rem <= acc + n) { gsel = c; acc_at = acc; }
      acc += n;
    }
    acc = acc_at;
    uint32_t hb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t v = 0;
#pragma unroll
      for (int c = 0; c < 8; ++c) v = c == gsel ? h[4 * c + e] : v;
      hb[e] = (v >> half) & 0xFFFFu;
    }
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      if (acc < rem && rem <= acc + hb[e]) {
        out[3 * b] = (uint32_t)(base + 4 * gsel + e); out[3 * b + 1] = rem - acc; out[3 * b + 2] = hb[e];
      }
      acc += hb[e];
    }
  }
}

template <int NT, int KPT, bool LO>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  constexpr int NW = NT / 64;
  constexpr int kBins = 2048;
  __shared__ __align__(16) uint32_t hist[3][kBins + 4];   // one per pass; bin kBins: not counted
  __shared__ uint32_t cnt[2][KPT][NW];      // ballot counts of the two ordered scans
  __shared__ uint32_t wsum[2][NW];          // per wave: OR of eligible keys, eligible count
  __shared__ uint32_t found[8];             // hi: digit, rem, count; lo: digit, rem, count
  __shared__ uint32_t ckey[kMaxClusters];   // cluster keys (cluster > 1)

  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const size_t roff = (size_t)row * a.ld;

  // ---- keys; every load is issued before the first use
  uint32_t key[KPT];
  const uint32_t* kp = reinterpret_cast<const uint32_t*>(a.keys) + roff;
  if (a.cluster == 1) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = j * NT + t < a.n ? kp[j * NT + t] : 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = key_of_bits(a.key_type, key[j]);
  } else {
    // cluster keys: coalesced reads of the n*cluster values, max per cluster
    // in LDS (the value index i belongs to cluster floor((i + 0.5) / cluster),
    // exact in fp32 for these sizes)
    for (int c = t; c < a.n; c += NT) ckey[c] = 0u;
    __syncthreads();
    const int total = a.n * a.cluster;
    const float inv = 1.0f / (float)a.cluster;
    if ((a.cluster & 3) == 0 && (a.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(a.keys) & 15) == 0) {
      // 4 values of one cluster per load; 8 loads in flight per thread
      for (int i0 = 4 * t; i0 < total; i0 += 32 * NT) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + 4 * NT * u;
          v[u] = i < total ? *reinterpret_cast<const uint4*>(kp + i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + 4 * NT * u;
          const uint32_t m =
              max(max(key_of_bits(a.key_type, v[u].x), key_of_bits(a.key_type, v[u].y)),
                  max(key_of_bits(a.key_type, v[u].z), key_of_bits(a.key_type, v[u].w)));
          if (i < total && m) atomicMax(&ckey[(int)(((float)i + 0.5f) * inv)], m);
        }
      }
    } else {
      for (int i0 = t; i0 < total; i0 += 8 * NT) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i0 + NT * u < total ? kp[i0 + NT * u] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + NT * u;
          const uint32_t m = key_of_bits(a.key_type, v[u]);
          if (i < total && m) atomicMax(&ckey[(int)(((float)i + 0.5f) * inv)], m);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = j * NT + t < a.n ? ckey[j * NT + t] : 0u;
  }
  uint32_t elig = 0, kor = 0, ecount = 0;   // bit j: entry j*NT+t takes part
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool e = (j * NT + t < a.n) & (!a.nonzero_only | (key[j] != 0u));
    elig |= (e ? 1u : 0u) << j;
    kor |= e ? key[j] : 0u;
    if (a.nonzero_only) ecount += (uint32_t)__popcll(__ballot(e));   // else every entry counts
  }
  kor = wave_incl<true>(kor);
  if (lane == 63) { wsum[0][w] = kor; wsum[1][w] = ecount; }
  // the first pass's histogram now; the later passes' ones while wave 0 scans the first
  for (int i = t; i < kBins + 4; i += NT) hist[0][i] = 0u;
  __syncthreads();

  uint32_t all_or = 0, E = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) { all_or |= wsum[0][i]; E += wsum[1][i]; }
  if (!a.nonzero_only) E = (uint32_t)a.n;
  const uint32_t rhi = min((uint32_t)a.r_hi, E);
  const uint32_t rlo = LO ? min((uint32_t)a.r_lo, rhi) : 0u;
  // all_hi / all_lo: the bound covers every eligible entry (no search)
  const bool all_hi = rhi == E;
  const bool all_lo = rlo == E && rlo > 0;
  const bool need_hi = rhi > 0 && !all_hi;
  const bool need_lo = rlo > 0 && !all_lo;

  // T_r (pre_*), rank left among the keys equal to T_r (rem_*), their count (tie_*)
  uint32_t pre_hi = 0, pre_lo = 0, rem_hi = rhi, rem_lo = rlo, tie_hi = E, tie_lo = E;
  if (need_hi || need_lo) {
    const int msb = all_or ? 31 - __builtin_clz(all_or) : -1;
    int lo_bit = msb + 1;                      // lowest bit decided so far
#pragma unroll 1
    for (int pass = 0; lo_bit > 0; ++pass) {
      const int width = lo_bit < 11 ? lo_bit : 11;
      const int shift = lo_bit - width;
      const uint32_t mask = (1u << width) - 1u;
      uint32_t* H = hist[pass];
      if (pass == 0) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const uint32_t bin = ((elig >> j) & 1u) ? (key[j] >> shift) & mask : (uint32_t)kBins;
          atomicAdd(&H[bin], 0x10001u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const uint32_t k = key[j];
          const bool e = (elig >> j) & 1u;
          const bool mh = e && need_hi && (k >> lo_bit) == (pre_hi >> lo_bit);
          const bool ml = e && need_lo && (k >> lo_bit) == (pre_lo >> lo_bit);
          const uint32_t inc = (mh ? 0x10000u : 0u) + (ml ? 1u : 0u);
          if (inc) atomicAdd(&H[(k >> shift) & mask], inc);
        }
      }
      __syncthreads();
      if (w == 0) {
        scan_pass(H, 1 << width, need_hi, rem_hi, need_lo, rem_lo, found);
      } else if (pass == 0) {
        for (int i = t - 64; i < 2 * (kBins + 4); i += NT - 64) (&hist[1][0])[i] = 0u;
      }
      __syncthreads();
      // found[] is written again only after the next pass's histogram
      // barrier, which every thread reaches after these reads
      if (need_hi) { pre_hi |= found[0] << shift; rem_hi = found[1]; tie_hi = found[2]; }
      if (need_lo) { pre_lo |= found[3] << shift; rem_lo = found[4]; tie_lo = found[5]; }
      lo_bit = shift;
    }
  }

  // ---- ties: rank the entries equal to T_r only when the bound splits them
  const bool split_hi = need_hi && tie_hi > rem_hi;
  const bool split_lo = need_lo && tie_lo > rem_lo;
  uint32_t eq_h = 0, eq_l = 0, eq_off = 0;
  if (split_hi || split_lo) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool e = (elig >> j) & 1u;
      eq_h |= ((e && split_hi && key[j] == pre_hi) ? 1u : 0u) << j;
      eq_l |= ((e && split_lo && key[j] == pre_lo) ? 1u : 0u) << j;
    }
    ordered_counts<NT, KPT, LO>(eq_h, eq_l, cnt[0]);
    __syncthreads();
    uint32_t dummy;
    eq_off = ordered_offsets<NT, KPT>(cnt[0], dummy);
  }

  uint32_t sel = 0, top = 0;   // bit j: entry j*NT+t is selected / in the top list
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int n = j * NT + t;
    const uint32_t k = key[j];
    const bool e = (elig >> j) & 1u;
    uint32_t eqpos = 0;
    if (split_hi || split_lo)
      eqpos = ordered_pos<LO>((uint32_t)__builtin_amdgcn_readlane((int)eq_off, j), eq_h, eq_l, j);
    const bool gt_hi = (k > pre_hi) | ((k == pre_hi) & ((eqpos >> 16) < rem_hi));
    const bool gt_lo = (k > pre_lo) | ((k == pre_lo) & ((eqpos & 0xFFFFu) < rem_lo));
    const bool in_hi = e & (all_hi | (need_hi & gt_hi));
    const bool in_lo = e & (all_lo | (need_lo & gt_lo));
    bool s = in_hi & !in_lo;
    if (a.include_mask && n < a.n) s |= a.include_mask[n] != 0;
    sel |= (s ? 1u : 0u) << j;
    top |= (in_lo ? 1u : 0u) << j;
  }

  // one ordered scan for both lists: selected in the high half, top list in the low
  ordered_counts<NT, KPT, LO>(sel, top, cnt[1]);
  __syncthreads();
  uint32_t total;
  const uint32_t off = ordered_offsets<NT, KPT>(cnt[1], total);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int n = j * NT + t;
    const uint32_t pos = ordered_pos<LO>((uint32_t)__builtin_amdgcn_readlane((int)off, j), sel, top, j);
    const bool s = (sel >> j) & 1u;
    if (n < a.n) {
      if (a.mask_out) a.mask_out[(size_t)row * a.ld_mask + n] = s ? 1 : 0;
      if (s) {
        if (a.idx_out) a.idx_out[(size_t)row * a.ld_idx + (pos >> 16)] = n;
        if (a.freq) atomicAdd(&a.freq[n], 1u);
      }
      if (((top >> j) & 1u) && a.idx_top_out)
        a.idx_top_out[(size_t)row * a.ld_idx_top + (pos & 0xFFFFu)] = n;
    }
  }
  if (t == 0 && a.count_out) a.count_out[row] = (int32_t)(total >> 16);
  if (t == 0 && a.count_top_out) a.count_top_out[row] = (int32_t)(total & 0xFFFFu);
}

template <int NT, bool LO>
static hipError_t launch_nt(const SelectArgs& a, hipStream_t s) {
  const int need = (a.n + NT - 1) / NT;
  dim3 grid(a.rows), block(NT);
  if (need <= 1) hipLaunchKernelGGL((select_kernel<NT, 1, LO>), grid, block, 0, s, a);
  else if (need <= 2) hipLaunchKernelGGL((select_kernel<NT, 2, LO>), grid, block, 0, s, a);
  else if (need <= 4) hipLaunchKernelGGL((select_kernel<NT, 4, LO>), grid, block, 0, s, a);
  else if (need <= 8) hipLaunchKernelGGL((select_kernel<NT, 8, LO>), grid, block, 0, s, a);
  else if (need <= 16) hipLaunchKernelGGL((select_kernel<NT, 16, LO>), grid, block, 0, s, a);
  else if (need <= 20) hipLaunchKernelGGL((select_kernel<NT, 20, LO>), grid, block, 0, s, a);
  else if (need <= 24) hipLaunchKernelGGL((select_kernel<NT, 24, LO>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((select_kernel<NT, 32, LO>), grid, block, 0, s, a);
  return hipGetLastError();
}

// Ranges that start at rank 0 (no lower bound, no second list) take the
// variant that carries one ballot per entry instead of two.
template <int NT>
static hipError_t launch_nt(const SelectArgs& a, hipStream_t s) {
  return a.r_lo > 0 ? launch_nt<NT, true>(a, s) : launch_nt<NT, false>(a, s);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  // Small rows take 256 threads (cheaper barriers); from 1024 entries on,
  // 1024 threads (up to 32 entries each) spread the histogram atomics.
  // Cluster mode reads n*cluster values: 1024 threads keep more loads in flight.
  if (a.n <= 1024 && (long)a.n * a.cluster <= 1024) return launch_nt<256>(a, s);
  return launch_nt<1024>(a, s);
}

}  // namespace sffn
