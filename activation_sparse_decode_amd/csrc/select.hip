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
// With a key scale vector, the key of entry j is the magnitude key of the
// fp32 product v_j * scale_j, formed as the keys are loaded (WiSparse's
// weight-aware saliency: activation magnitude times a precomputed weight
// norm of the channel).  With clear_keys the row's keys are set to zero
// once read (a frequency count consumed and reset in the same pass).
// Entries marked in an exclusion mask take no part
// in the ranking; with the same mask as the include mask the call yields
// "the set, then the best-ranked entries outside it until k more": the
// secondary neurons added to the base set until the loading budget is met
// (SelectInfer §4, Fig 6) and the dynamic neurons added to the static ones
// until the computed fraction is reached (§5).
//
// Method: NT threads; wave w owns the KPT*64 consecutive entries starting at
// w*KPT*64, lane l the entries w*KPT*64 + j*64 + l (j < KPT), so every load
// and every mask store of a wave is contiguous.  One workgroup handles a row
// (at most 32768 entries): the cost is the instructions each wave issues
// and the chain of barriers, and the kernel keeps both short.
//  1. The largest eligible key (an OR over the row) fixes the most
//     significant bit that varies, so the digits start there: keys that fit
//     in 11 bits (e.g. frequency counts) take one pass, float magnitudes 3.
//  2. MSB-first radix search finds, for each bound r in {r_hi, r_lo}, the key
//     T_r of the r-th largest entry, how many entries equal to T_r fall
//     inside the top r, and how many equal T_r in all.  Both bounds share
//     one LDS histogram (16-bit halves of one counter).  Entries that take no
//     part count into per-lane sink bins that are never read: LDS atomics of
//     one wave on one address serialise, so a shared sink would cost ~2
//     cycles per lane.  Every thread scans its share of the bins (counts
//     above it from a DPP scan within the wave plus the totals of the waves
//     before), and the one thread whose bins hold the rank walks them.
//     After the first pass only the keys whose higher digits match a bound
//     can matter: each thread tests its own keys and only those are
//     counted.  A bound that covers every eligible entry needs no search
//     (pure compaction, e.g. the nonzero clusters of a ReLU layer), and a
//     bound whose boundary digit holds exactly the entries still needed
//     stops there: every key with that prefix or a larger one is in (for
//     float magnitudes usually after the second pass, saving the third).
//  3. Index-order positions: a wave's entries are consecutive, so the
//     position of an entry among those with some property is the count in
//     the waves before (one exchange through LDS), plus the wave's running
//     count over its earlier slots (scalar bit counts of ballots), plus the
//     lower lanes of its own ballot.  This places the selected indices
//     (ascending lists, contiguous stores) and, when T_r is tied across the
//     bound, ranks the tied entries in index order, which decides them as the
//     (key desc, index asc) order does.
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

// One radix pass's scan over nb bins (nb a power of two <= kBins), done by
// all NT threads: thread t holds the c = max(1, nb/NT) bins [nb-(t+1)c,
// nb-tc) (thread 0 the largest digits).  For each bound it writes the digit
// holding rank `rem` (in the packed counters' hi or lo half), the rank left
// inside that digit and the digit's count to out[3b..3b+2].  WT: NT/64
// words of LDS.  Starts after the barrier that completes H; ends with a
// barrier after which out[] is valid.
template <int NT>
__device__ __forceinline__ void scan_pass(const uint32_t* H, int nb, bool want_hi, uint32_t rem_hi,
                                          bool want_lo, uint32_t rem_lo, uint32_t* WT,
                                          uint32_t* out) {
  constexpr int NW = NT / 64;
  constexpr int CB = 2048 / NT;   // most bins a thread holds
  const int t = threadIdx.x, lane = t & 63, w = wave_id();
  const int c = nb >= NT ? nb / NT : 1;
  const int base = nb - (t + 1) * c;
  uint32_t h[CB];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    h[i] = (i < c && base >= 0) ? H[base + i] : 0u;
    own += h[i];
  }
  const uint32_t incl = wave_incl<false>(own);
  if (lane == 63) WT[w] = incl;
  __syncthreads();
  uint32_t above = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) above += ww < w ? WT[ww] : 0u;
  above += incl - own;   // packed count of the bins above this thread's
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const bool want = b == 0 ? want_hi : want_lo;
    const int half = b == 0 ? 16 : 0;
    const uint32_t rem = b == 0 ? rem_hi : rem_lo;
    const uint32_t a0 = (above >> half) & 0xFFFFu;
    if (!(want && a0 < rem && rem <= a0 + ((own >> half) & 0xFFFFu))) continue;   // one thread
    uint32_t acc = a0;
#pragma unroll
    for (int i = CB - 1; i >= 0; --i) {
      if (i >= c) continue;
      const uint32_t hb = (h[i] >> half) & 0xFFFFu;
      if (acc < rem && rem <= acc + hb) {
        out[3 * b] = (uint32_t)(base + i); out[3 * b + 1] = rem - acc; out[3 * b + 2] = hb;
      }
      acc += hb;
    }
  }
  __syncthreads();
}

// Sum over the waves before this one (and over all waves) of a packed
// per-wave count that lane 0 of each wave stored in WT.  Call after the
// barrier that follows the stores.
template <int NW>
__device__ __forceinline__ uint32_t waves_before(const uint32_t* WT, uint32_t& total) {
  const int w = wave_id();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) {
    const uint32_t v = WT[ww];
    before += ww < w ? v : 0u;
    all += v;
  }
  total = all;
  return before;
}

template <int NT, int KPT, bool LO>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  constexpr int NW = NT / 64;
  constexpr int kBins = 2048;
  constexpr int kHist = kBins + 64;   // bins kBins + lane: sinks of pass 0, never read
  __shared__ __align__(16) uint32_t hist[3][kHist];   // one per pass
  __shared__ uint32_t WT[4][NW];            // per-wave words: scans, ties, list counts
  __shared__ uint32_t wsum[2][NW];          // per wave: OR of eligible keys, eligible count
  __shared__ uint32_t found[8];             // hi: digit, rem, count; lo: digit, rem, count
  __shared__ uint32_t ckey[kMaxClusters];   // cluster keys (cluster > 1)

  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, w = wave_id();
  const size_t roff = (size_t)row * a.ld;
  const int ebase = w * KPT * 64 + lane;   // entry of slot j: ebase + 64 j
  const int n = a.n;

  // ---- keys; every load is issued before the first use (clamped addresses,
  // no branch around a load)
  uint32_t key[KPT];
  const uint32_t* kp = reinterpret_cast<const uint32_t*>(a.keys) + roff;
  if (a.cluster == 1) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = kp[min(ebase + 64 * j, n - 1)];
    if (a.key_scale) {
      // weight-aware magnitude: the key of the fp32 product v_j * scale_j
      float sc[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) sc[j] = a.key_scale[min(ebase + 64 * j, n - 1)];
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        key[j] = ebase + 64 * j < n ? key_abs(__uint_as_float(key[j]) * sc[j]) : 0u;
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        key[j] = ebase + 64 * j < n ? key_of_bits(a.key_type, key[j]) : 0u;
    }
  } else {
    // cluster keys: coalesced reads of the n*cluster values, max per cluster
    // in LDS (value i belongs to cluster i / cluster, an exact unsigned
    // integer division for every accepted cluster size)
    for (int c = t; c < n; c += NT) ckey[c] = 0u;
    __syncthreads();
    const int total = n * a.cluster;
    const uint32_t csz = (uint32_t)a.cluster;
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
          if (i < total && m) atomicMax(&ckey[(uint32_t)i / csz], m);
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
          if (i < total && m) atomicMax(&ckey[(uint32_t)i / csz], m);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = ebase + 64 * j < n ? ckey[ebase + 64 * j] : 0u;
  }
  uint32_t incl = 0;   // bit j: entry of slot j is in include_mask (clamped reads)
  if (a.include_mask) {
    uint8_t incm[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) incm[j] = a.include_mask[min(ebase + 64 * j, n - 1)];
#pragma unroll
    for (int j = 0; j < KPT; ++j) incl |= (((ebase + 64 * j < n) & (incm[j] != 0)) ? 1u : 0u) << j;
  }
  uint32_t excl = 0;   // bit j: entry of slot j is in exclude_mask (clamped reads)
  if (a.exclude_mask) {
    uint8_t exm[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) exm[j] = a.exclude_mask[min(ebase + 64 * j, n - 1)];
#pragma unroll
    for (int j = 0; j < KPT; ++j) excl |= (exm[j] != 0 ? 1u : 0u) << j;
  }

  uint32_t elig = 0, kor = 0;   // bit j: entry of slot j takes part
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool e = (ebase + 64 * j < n) & (!a.nonzero_only | (key[j] != 0u)) & !((excl >> j) & 1u);
    elig |= (e ? 1u : 0u) << j;
    kor |= e ? key[j] : 0u;
  }
  if (a.clear_keys) {
    // the keys were consumed above (their loads have completed): reset the
    // row's own entries, so a frequency count can be read and cleared in one pass
    uint32_t* kw = const_cast<uint32_t*>(kp);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (ebase + 64 * j < n) kw[ebase + 64 * j] = 0u;
  }
  kor = wave_incl<true>(kor);
  const uint32_t ecount = wave_incl<false>((uint32_t)__popc(elig));   // lane 63: the wave's count
  if (lane == 63) { wsum[0][w] = kor; wsum[1][w] = ecount; }
  // all three histograms (the sinks are never read)
  {
    uint4* hz = reinterpret_cast<uint4*>(&hist[0][0]);
    for (int i = t; i < 3 * kHist / 4; i += NT) hz[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();

  uint32_t all_or = 0, E = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) { all_or |= wsum[0][i]; E += wsum[1][i]; }
  if (!a.nonzero_only && !a.exclude_mask) E = (uint32_t)n;
  const uint32_t rhi = min((uint32_t)a.r_hi, E);
  const uint32_t rlo = LO ? min((uint32_t)a.r_lo, rhi) : 0u;
  // all_hi / all_lo: the bound covers every eligible entry (no search)
  const bool all_hi = rhi == E;
  const bool all_lo = rlo == E && rlo > 0;
  bool need_hi = rhi > 0 && !all_hi;
  bool need_lo = rlo > 0 && !all_lo;

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
          const uint32_t bin = ((elig >> j) & 1u) ? (key[j] >> shift) & mask : (uint32_t)(kBins + lane);
          atomicAdd(&H[bin], 0x10001u);
        }
      } else {
        // only keys whose decided digits match a bound's count; a bound that
        // is not searched compares against a value no shifted key reaches
        const uint32_t ph = need_hi ? pre_hi >> lo_bit : 0xFFFFFFFFu;
        const uint32_t pl = need_lo ? pre_lo >> lo_bit : 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
          const uint32_t k = key[j];
          const uint32_t inc = ((k >> lo_bit) == ph ? 0x10000u : 0u) + ((k >> lo_bit) == pl ? 1u : 0u);
          if (inc) atomicAdd(&H[(k >> shift) & mask], inc);
        }
      }
      __syncthreads();
      scan_pass<NT>(H, 1 << width, need_hi, rem_hi, need_lo, rem_lo, WT[0], found);
      // found[] is written again only after the next pass's first barrier
      // inside scan_pass, which every thread reaches after these reads
      if (need_hi) { pre_hi |= found[0] << shift; rem_hi = found[1]; tie_hi = found[2]; }
      if (need_lo) { pre_lo |= found[3] << shift; rem_lo = found[4]; tie_lo = found[5]; }
      // A bound whose boundary digit holds exactly the entries still needed
      // is decided: every key whose prefix is at least pre_* is in, whatever
      // its lower bits (pre_* has zeros there), so its search stops.
      if (need_hi && tie_hi == rem_hi) need_hi = false;
      if (need_lo && tie_lo == rem_lo) need_lo = false;
      if (pass == 0 && shift > 0) {
        // Entries that take no part get a key whose first digit is neither
        // bound's (the first digit has 11 bits when more passes follow), so
        // the later passes need no eligibility test.
        const uint32_t dh = need_hi ? pre_hi >> shift : 0xFFFFFFFFu;
        const uint32_t dl = need_lo ? pre_lo >> shift : 0xFFFFFFFFu;
        const uint32_t d = (dh != 0u && dl != 0u) ? 0u : (dh != 1u && dl != 1u) ? 1u : 2u;
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = ((elig >> j) & 1u) ? key[j] : d << shift;
      }
      lo_bit = shift;
      if (!need_hi && !need_lo) break;   // uniform: found[] is shared
    }
  }

  if (a.thr_out) {
    // Threshold mode (every entry eligible, no lists): for the range [0, r_hi)
    // the key T and the index I of the last entry equal to T inside -- entry j
    // is in iff key_j > T, or key_j == T and j <= I -- and, with thr_top_out,
    // the same pair for [0, r_lo).  Without a split tie every entry whose key
    // reaches the decided prefix is in (I = INT_MAX).
    uint32_t* th = a.thr_out + 2 * (size_t)row;
    uint32_t* tl = a.thr_top_out ? a.thr_top_out + 2 * (size_t)row : nullptr;
    const bool split_h = need_hi && tie_hi > rem_hi;
    const bool split_l = LO && need_lo && tie_lo > rem_lo;
    if (t == 0) {
      th[0] = rhi > 0 ? (all_hi ? 0u : pre_hi) : 0xFFFFFFFFu;
      if (!split_h) th[1] = rhi > 0 ? 0x7FFFFFFFu : 0xFFFFFFFFu;
      if (tl) {
        tl[0] = rlo > 0 ? (all_lo ? 0u : pre_lo) : 0xFFFFFFFFu;
        if (!split_l) tl[1] = rlo > 0 ? 0x7FFFFFFFu : 0xFFFFFFFFu;
      }
    }
    if (!(split_h || split_l)) return;
    // the entries equal to a split T in index order (hi: high half, lo: low
    // half of the packed counts): the rem-th is the last one inside
    uint32_t eq_h = 0, eq_l = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      eq_h |= (split_h && key[j] == pre_hi ? 1u : 0u) << j;
      eq_l |= (split_l && key[j] == pre_lo ? 1u : 0u) << j;
    }
    eq_h &= elig;
    eq_l &= elig;
    const uint32_t wc = wave_incl<false>(((uint32_t)__popc(eq_h) << 16) + (uint32_t)__popc(eq_l));
    if (lane == 63) WT[1][w] = wc;
    __syncthreads();
    uint32_t dummy;
    uint32_t eq_run = waves_before<NW>(WT[1], dummy);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint64_t bh = __ballot((eq_h >> j) & 1u);
      const uint64_t bl = __ballot((eq_l >> j) & 1u);
      const uint32_t ph = (eq_run >> 16) + lanes_below(bh), pl = (eq_run & 0xFFFFu) + lanes_below(bl);
      eq_run += ((uint32_t)__popcll(bh) << 16) + (uint32_t)__popcll(bl);
      if (((eq_h >> j) & 1u) && ph + 1u == rem_hi) th[1] = (uint32_t)(ebase + 64 * j);
      if (((eq_l >> j) & 1u) && pl + 1u == rem_lo && tl) tl[1] = (uint32_t)(ebase + 64 * j);
    }
    return;
  }

  // ---- membership of the two rank ranges (before eligibility): bit j of
  // hib / lob: the entry of slot j is among the top r_hi / top r_lo.  When a
  // bound splits the entries equal to T_r, those are ranked in index order.
  const bool split_hi = need_hi && tie_hi > rem_hi;
  const bool split_lo = need_lo && tie_lo > rem_lo;
  const uint32_t th_hi = all_hi ? 0u : pre_hi;   // no split: every tied entry is inside
  const uint32_t th_lo = all_lo ? 0u : pre_lo;
  uint32_t hib = 0, lob = 0;
  if (!(split_hi || split_lo)) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      hib |= (key[j] >= th_hi ? 1u : 0u) << j;
      if (LO) lob |= (key[j] >= th_lo ? 1u : 0u) << j;
    }
  } else {
    uint32_t eq_h = 0, eq_l = 0;   // bit j: eligible and equal to a split T_r
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      eq_h |= (split_hi && key[j] == pre_hi ? 1u : 0u) << j;
      eq_l |= (split_lo && key[j] == pre_lo ? 1u : 0u) << j;
    }
    eq_h &= elig;
    eq_l &= elig;
    const uint32_t wc = wave_incl<false>(((uint32_t)__popc(eq_h) << 16) + (uint32_t)__popc(eq_l));
    if (lane == 63) WT[1][w] = wc;
    __syncthreads();
    uint32_t dummy;
    uint32_t eq_run = waves_before<NW>(WT[1], dummy);   // equal entries in earlier waves
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t k = key[j];
      const uint64_t bh = __ballot((eq_h >> j) & 1u);
      const uint64_t bl = __ballot((eq_l >> j) & 1u);
      const uint32_t pos = eq_run + ((lanes_below(bh) << 16) | lanes_below(bl));
      eq_run += ((uint32_t)__popcll(bh) << 16) + (uint32_t)__popcll(bl);
      const bool gh = split_hi ? (k > pre_hi) | ((k == pre_hi) & ((pos >> 16) < rem_hi)) : k >= th_hi;
      const bool gl = split_lo ? (k > pre_lo) | ((k == pre_lo) & ((pos & 0xFFFFu) < rem_lo)) : k >= th_lo;
      hib |= (gh ? 1u : 0u) << j;
      if (LO) lob |= (gl ? 1u : 0u) << j;
    }
  }
  hib = rhi > 0 ? hib & elig : 0u;
  lob = LO && rlo > 0 ? lob & elig : 0u;
  const uint32_t sel = (hib & ~lob) | incl;   // bit j: selected
  const uint32_t top = lob;                   // bit j: in the top list

  // ---- per-wave counts (selected: hi half, top list: lo half), then the
  // counts of the waves before
  {
    const uint32_t wc = wave_incl<false>(((uint32_t)__popc(sel) << 16) + (uint32_t)__popc(top));
    if (lane == 63) WT[2][w] = wc;
  }
  __syncthreads();
  uint32_t total;
  uint32_t run = waves_before<NW>(WT[2], total);

  // ---- stores; index lists: positions in index order, contiguous within
  // each ballot
  int eb = ebase;
  asm volatile("" : "+v"(eb));   // bounds tests made again here, not kept live since the loads
  int32_t* irow = a.idx_out ? a.idx_out + (size_t)row * a.ld_idx : nullptr;
  int32_t* trow = (LO && a.idx_top_out) ? a.idx_top_out + (size_t)row * a.ld_idx_top : nullptr;
  if (irow || trow) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int e = eb + 64 * j;
      const bool sj = (sel >> j) & 1u;
      const bool tj = LO && ((top >> j) & 1u);
      const uint64_t bs = __ballot(sj);
      const uint64_t bt = LO ? __ballot(tj) : 0ull;
      const uint32_t ps = (run >> 16) + lanes_below(bs);
      const uint32_t pt = (run & 0xFFFFu) + lanes_below(bt);
      run += ((uint32_t)__popcll(bs) << 16) + (uint32_t)__popcll(bt);
      if (irow && sj) irow[ps] = e;
      if (trow && tj) trow[pt] = e;
    }
  }
  if (a.mask_out) {
    uint8_t* mrow = a.mask_out + (size_t)row * a.ld_mask;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int e = eb + 64 * j;
      if (e < n) mrow[e] = (uint8_t)((sel >> j) & 1u);
    }
  }
  if (a.freq) {
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if ((sel >> j) & 1u) atomicAdd(&a.freq[eb + 64 * j], 1u);
  }
  if (t == 0 && a.count_out) a.count_out[row] = (int32_t)(total >> 16);
  if (t == 0 && a.count_top_out) a.count_top_out[row] = (int32_t)(total & 0xFFFFu);
}

template <int NT, bool LO, int... K>
struct SelectLaunch;

template <int NT, bool LO, int K0, int... K>
struct SelectLaunch<NT, LO, K0, K...> {
  static hipError_t go(const SelectArgs& a, hipStream_t s) {
    if (sizeof...(K) == 0 || a.n <= NT * K0) {
      hipLaunchKernelGGL((select_kernel<NT, K0, LO>), dim3(a.rows), dim3(NT), 0, s, a);
      return hipGetLastError();
    }
    return SelectLaunch<NT, LO, K...>::go(a, s);
  }
};
template <int NT, bool LO>
struct SelectLaunch<NT, LO> {
  static hipError_t go(const SelectArgs&, hipStream_t) { return hipErrorInvalidValue; }
};

// Entries per lane: the smallest listed count that covers the row, so few
// slots are dead.  Ranges that start at rank 0 (no lower bound, no second
// list) take the variant with one list.
template <bool LO>
static hipError_t launch_lo(const SelectArgs& a, hipStream_t s) {
  // Small rows take 256 threads (cheaper barriers), rows up to 4096 entries
  // 512 threads, longer rows 1024 threads (up to 32 entries each) over 16
  // waves (measured on MI355X: 4096 keys 7.8 us at 512 threads vs 8.2 at
  // 1024; 8192 and 14336 keys faster at 1024).  Cluster mode reads
  // n*cluster values: 1024 threads keep more loads in flight.
  if (a.n <= 1024 && (long)a.n * a.cluster <= 1024) return SelectLaunch<256, LO, 1, 2, 4>::go(a, s);
  if (a.n <= 4096 && a.cluster == 1) return SelectLaunch<512, LO, 4, 6, 8>::go(a, s);
  return SelectLaunch<1024, LO, 1, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20, 24, 28, 32>::go(a, s);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  return a.r_lo > 0 ? launch_lo<true>(a, s) : launch_lo<false>(a, s);
}

}  // namespace sffn
