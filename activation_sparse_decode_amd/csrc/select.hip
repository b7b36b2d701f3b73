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
// Method: NT threads; thread t owns the KPT consecutive entries
// [t*KPT, (t+1)*KPT) in registers, so thread order is index order.
//  1. MSB-first radix search (digits of 11, 11 and 10 bits, LDS histograms)
//     finds, for each bound r in {r_hi, r_lo}, the key T_r of the r-th
//     largest entry and how many entries equal to T_r fall inside the top r.
//     Both searches share one histogram (16-bit halves of one counter).  A
//     bound that covers every eligible entry needs no search (pure
//     compaction, e.g. the nonzero clusters of a ReLU layer).
//  2. An exclusive scan of per-thread "key == T_r" counts gives every entry
//     its rank among equal keys in index order, which decides the ties
//     exactly as the (key desc, index asc) order does.
//  3. Exclusive scans of the selected counts give output positions: the
//     compacted index lists come out ascending.
// Everything is integer: the result is unique and bit-exact.
#include "sffn_device.h"

namespace sffn {

template <int NW>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[w] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t s = tmp[i];
    before += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

__device__ __forceinline__ uint32_t key_of_bits(int key_type, uint32_t b) {
  if (key_type == 0) return b & 0x7FFFFFFFu;
  if (key_type == 1) return b;
  return key_signed(__uint_as_float(b));
}

__device__ __forceinline__ uint32_t make_key(const SelectArgs& a, size_t off) {
  return key_of_bits(a.key_type, reinterpret_cast<const uint32_t*>(a.keys)[off]);
}

template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t tmp[NW];
  __shared__ uint32_t found[4];   // digit_hi, rem_hi, digit_lo, rem_lo

  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int base = t * KPT;
  const size_t roff = (size_t)row * a.ld;

  uint32_t key[KPT];
  uint32_t elig = 0;   // bit j: entry base+j takes part
  // 16-byte loads when a thread's four consecutive keys are aligned and in range
  const bool vec = KPT % 4 == 0 && a.cluster == 1 && (a.ld & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.keys) & 15) == 0;
#pragma unroll
  for (int j4 = 0; j4 < KPT; j4 += 4) {
    if (vec && base + j4 + 3 < a.n) {
      const uint4 v = *reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint32_t*>(a.keys) + roff + base + j4);
      const uint32_t b[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4 && j4 + e < KPT; ++e) key[j4 + e] = key_of_bits(a.key_type, b[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4 && j4 + e < KPT; ++e) {
        const int n = base + j4 + e;
        uint32_t k = 0;
        if (n < a.n) {
          if (a.cluster == 1) {
            k = make_key(a, roff + n);
          } else {
            const size_t c0 = roff + (size_t)n * a.cluster;
            for (int g = 0; g < a.cluster; ++g) {
              const uint32_t v = make_key(a, c0 + g);
              k = v > k ? v : k;
            }
          }
        }
        key[j4 + e] = k;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (base + j < a.n && (!a.nonzero_only || key[j] != 0u)) elig |= 1u << j;

  uint32_t E;
  block_excl_scan<NW>((uint32_t)__popc(elig), tmp, E);
  const int rhi = min(a.r_hi, (int)E);
  const int rlo = min(a.r_lo, rhi);
  // all_hi / all_lo: the bound covers every eligible entry (no search)
  const bool all_hi = rhi == (int)E;
  const bool all_lo = rlo == (int)E && rlo > 0;
  const bool need_hi = rhi > 0 && !all_hi;
  const bool need_lo = rlo > 0 && !all_lo;

  uint32_t pre_hi = 0, pre_lo = 0;
  uint32_t rem_hi = (uint32_t)rhi, rem_lo = (uint32_t)rlo;

  if (need_hi || need_lo) {
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int bits = pass == 2 ? 10 : 11;
      const int nb = 1 << bits;
      const int top = shift + bits;   // bits above this digit are decided
      for (int i = t; i < nb; i += NT) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if (elig & (1u << j)) {
          const uint32_t k = key[j];
          const bool mh = need_hi && (pass == 0 || (k >> top) == (pre_hi >> top));
          const bool ml = need_lo && (pass == 0 || (k >> top) == (pre_lo >> top));
          const uint32_t inc = (mh ? 0x10000u : 0u) + (ml ? 1u : 0u);
          if (inc) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], inc);
        }
      }
      __syncthreads();
      // thread t covers the digits nb-1-q*t .. nb-q*(t+1) (descending), q = nb/NT
      constexpr int Q = 2048 / NT;
      const int q = nb / NT > 0 ? nb / NT : 1;
      uint32_t h[Q];
      uint32_t own = 0;
#pragma unroll
      for (int i = 0; i < Q; ++i) {
        const int dgt = nb - 1 - (q * t + i);
        h[i] = (i < q && dgt >= 0 && q * t + i < nb) ? hist[dgt] : 0u;
        own += h[i];
      }
      uint32_t tot;
      const uint32_t above = block_excl_scan<NW>(own, tmp, tot);
      if (need_hi) {
        uint32_t acc = above >> 16;
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          const uint32_t c = h[i] >> 16;
          if (acc < rem_hi && rem_hi <= acc + c) {
            found[0] = (uint32_t)(nb - 1 - (q * t + i)); found[1] = rem_hi - acc;
          }
          acc += c;
        }
      }
      if (need_lo) {
        uint32_t acc = above & 0xFFFFu;
#pragma unroll
        for (int i = 0; i < Q; ++i) {
          const uint32_t c = h[i] & 0xFFFFu;
          if (acc < rem_lo && rem_lo <= acc + c) {
            found[2] = (uint32_t)(nb - 1 - (q * t + i)); found[3] = rem_lo - acc;
          }
          acc += c;
        }
      }
      __syncthreads();
      if (need_hi) { pre_hi |= found[0] << shift; rem_hi = found[1]; }
      if (need_lo) { pre_lo |= found[2] << shift; rem_lo = found[3]; }
      __syncthreads();
    }
  }

  // rank of each entry among the eligible entries equal to T_hi / T_lo
  uint32_t run_h = 0, run_l = 0;
  if (need_hi || need_lo) {
    uint32_t eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (elig & (1u << j)) {
        eq += (need_hi && key[j] == pre_hi) ? 0x10000u : 0u;
        eq += (need_lo && key[j] == pre_lo) ? 1u : 0u;
      }
    }
    uint32_t dummy;
    const uint32_t eq_before = block_excl_scan<NW>(eq, tmp, dummy);
    run_h = eq_before >> 16;
    run_l = eq_before & 0xFFFFu;
  }

  uint32_t sel = 0, sel_top = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int n = base + j;
    bool in_hi = false, in_lo = false;
    if (elig & (1u << j)) {
      const uint32_t k = key[j];
      if (all_hi) in_hi = true;
      else if (need_hi) {
        if (k > pre_hi) in_hi = true;
        else if (k == pre_hi) { in_hi = run_h < rem_hi; ++run_h; }
      }
      if (all_lo) in_lo = true;
      else if (need_lo) {
        if (k > pre_lo) in_lo = true;
        else if (k == pre_lo) { in_lo = run_l < rem_lo; ++run_l; }
      }
    }
    bool s = in_hi && !in_lo;
    if (a.include_mask && n < a.n && a.include_mask[n]) s = true;
    if (s) sel |= 1u << j;
    if (in_lo) sel_top |= 1u << j;
  }

  // one scan for both lists: selected count in the high half, top-list count in the low
  uint32_t total;
  const uint32_t pos2 = block_excl_scan<NW>(((uint32_t)__popc(sel) << 16) | (uint32_t)__popc(sel_top),
                                            tmp, total);
  uint32_t pos = pos2 >> 16, pos_top = pos2 & 0xFFFFu;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int n = base + j;
    if (n >= a.n) break;
    const bool s = (sel >> j) & 1u;
    if (a.mask_out) a.mask_out[(size_t)row * a.ld_mask + n] = s ? 1 : 0;
    if (s) {
      if (a.idx_out) a.idx_out[(size_t)row * a.ld_idx + pos] = n;
      ++pos;
      if (a.freq) atomicAdd(&a.freq[n], 1u);
    }
    if ((sel_top >> j) & 1u) {
      if (a.idx_top_out) a.idx_top_out[(size_t)row * a.ld_idx_top + pos_top] = n;
      ++pos_top;
    }
  }
  if (t == 0 && a.count_out) a.count_out[row] = (int32_t)(total >> 16);
  if (t == 0 && a.count_top_out) a.count_top_out[row] = (int32_t)(total & 0xFFFFu);
}

template <int NT>
static hipError_t launch_nt(const SelectArgs& a, hipStream_t s) {
  const int need = (a.n + NT - 1) / NT;
  dim3 grid(a.rows), block(NT);
  if (need <= 1) hipLaunchKernelGGL((select_kernel<NT, 1>), grid, block, 0, s, a);
  else if (need <= 2) hipLaunchKernelGGL((select_kernel<NT, 2>), grid, block, 0, s, a);
  else if (need <= 4) hipLaunchKernelGGL((select_kernel<NT, 4>), grid, block, 0, s, a);
  else if (need <= 8) hipLaunchKernelGGL((select_kernel<NT, 8>), grid, block, 0, s, a);
  else if (need <= 16) hipLaunchKernelGGL((select_kernel<NT, 16>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((select_kernel<NT, 32>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  // Fewer waves make every barrier and scan cheaper; 256 threads hold up
  // to 8192 entries (32 per thread), 1024 threads up to 32768.
  if (a.n <= 8192) return launch_nt<256>(a, s);
  return launch_nt<1024>(a, s);
}

}  // namespace sffn
