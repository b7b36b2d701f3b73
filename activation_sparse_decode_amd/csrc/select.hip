// Rank-range selection and compaction (one workgroup per row).
//
// The entries of a row are ordered by (key descending, index ascending) and
// the ranks [r_lo, r_hi) are selected: per-token top-alpha, top-beta by
// frequency and the top-delta base set of SelectInfer (§4, §5) are ranges
// [0, k); the SpAx middle tier (Fig 2) is [k_top, k_top + k_mid).
//
// Method: 1024 threads, thread t owns the KPT consecutive entries
// [t*KPT, (t+1)*KPT) in registers, so thread order is index order.
//  1. MSB-first radix search (digits of 11, 11 and 10 bits, LDS histograms)
//     finds, for each bound r in {r_hi, r_lo}, the key T_r of the r-th
//     largest entry and how many entries equal to T_r fall inside the top r.
//     Both searches share one histogram (16-bit halves of one counter).
//  2. An exclusive scan of per-thread "key == T_r" counts gives every entry
//     its rank among equal keys in index order, which decides the ties
//     exactly as the (key desc, index asc) order does.
//  3. An exclusive scan of the selected counts gives output positions: the
//     compacted index list comes out ascending.
// Everything is integer: the result is unique and bit-exact.
#include "sffn_device.h"

namespace sffn {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

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
  for (int i = 0; i < kSelWaves; ++i) {
    const uint32_t s = tmp[i];
    before += (i < w) ? s : 0u;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

template <int KPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t tmp[kSelWaves];
  __shared__ uint32_t found[4];   // digit_hi, rem_hi, digit_lo, rem_lo

  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int base = t * KPT;
  const size_t roff = (size_t)row * a.ld;

  uint32_t key[KPT];
  uint32_t elig = 0;   // bit j: entry base+j takes part
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int n = base + j;
    uint32_t k = 0;
    if (n < a.n) {
      if (a.key_type == 0) {
        k = __float_as_uint(reinterpret_cast<const float*>(a.keys)[roff + n]) & 0x7FFFFFFFu;
      } else if (a.key_type == 1) {
        k = reinterpret_cast<const uint32_t*>(a.keys)[roff + n];
      } else {
        k = key_signed(reinterpret_cast<const float*>(a.keys)[roff + n]);
      }
      if (!a.nonzero_only || k != 0u) elig |= 1u << j;
    }
    key[j] = k;
  }

  uint32_t E;
  block_excl_scan((uint32_t)__popc(elig), tmp, E);
  const int rhi = min(a.r_hi, (int)E);
  const int rlo = min(a.r_lo, rhi);
  const bool need_hi = rhi > 0;
  const bool need_lo = rlo > 0;

  uint32_t pre_hi = 0, pre_lo = 0;
  uint32_t rem_hi = (uint32_t)rhi, rem_lo = (uint32_t)rlo;

  if (need_hi) {
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int bits = pass == 2 ? 10 : 11;
      const int nb = 1 << bits;
      const int top = shift + bits;   // bits above this digit are decided
      for (int i = t; i < nb; i += kSelThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if (elig & (1u << j)) {
          const uint32_t k = key[j];
          const bool mh = pass == 0 || (k >> top) == (pre_hi >> top);
          const bool ml = need_lo && (pass == 0 || (k >> top) == (pre_lo >> top));
          const uint32_t inc = (mh ? 0x10000u : 0u) + (ml ? 1u : 0u);
          if (inc) atomicAdd(&hist[(k >> shift) & (uint32_t)(nb - 1)], inc);
        }
      }
      __syncthreads();
      // thread t covers digits nb-1-2t and nb-2-2t (descending)
      const bool own = 2 * t < nb;
      const uint32_t h0 = own ? hist[nb - 1 - 2 * t] : 0u;
      const uint32_t h1 = own ? hist[nb - 2 - 2 * t] : 0u;
      uint32_t tot;
      const uint32_t above = block_excl_scan(h0 + h1, tmp, tot);
      if (own) {
        const uint32_t ah = above >> 16, h0h = h0 >> 16, h1h = h1 >> 16;
        if (ah < rem_hi && rem_hi <= ah + h0h) {
          found[0] = (uint32_t)(nb - 1 - 2 * t); found[1] = rem_hi - ah;
        } else if (ah + h0h < rem_hi && rem_hi <= ah + h0h + h1h) {
          found[0] = (uint32_t)(nb - 2 - 2 * t); found[1] = rem_hi - ah - h0h;
        }
        if (need_lo) {
          const uint32_t al = above & 0xFFFFu, h0l = h0 & 0xFFFFu, h1l = h1 & 0xFFFFu;
          if (al < rem_lo && rem_lo <= al + h0l) {
            found[2] = (uint32_t)(nb - 1 - 2 * t); found[3] = rem_lo - al;
          } else if (al + h0l < rem_lo && rem_lo <= al + h0l + h1l) {
            found[2] = (uint32_t)(nb - 2 - 2 * t); found[3] = rem_lo - al - h0l;
          }
        }
      }
      __syncthreads();
      pre_hi |= found[0] << shift;
      rem_hi = found[1];
      if (need_lo) {
        pre_lo |= found[2] << shift;
        rem_lo = found[3];
      }
      __syncthreads();
    }
  }

  // rank of each entry among the eligible entries equal to T_hi / T_lo
  uint32_t eq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (elig & (1u << j)) {
      eq += (need_hi && key[j] == pre_hi) ? 0x10000u : 0u;
      eq += (need_lo && key[j] == pre_lo) ? 1u : 0u;
    }
  }
  uint32_t dummy;
  const uint32_t eq_before = block_excl_scan(eq, tmp, dummy);
  uint32_t run_h = eq_before >> 16, run_l = eq_before & 0xFFFFu;

  uint32_t sel = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int n = base + j;
    bool in_hi = false, in_lo = false;
    if (elig & (1u << j)) {
      const uint32_t k = key[j];
      if (need_hi) {
        if (k > pre_hi) in_hi = true;
        else if (k == pre_hi) { in_hi = run_h < rem_hi; ++run_h; }
      }
      if (need_lo) {
        if (k > pre_lo) in_lo = true;
        else if (k == pre_lo) { in_lo = run_l < rem_lo; ++run_l; }
      }
    }
    bool s = in_hi && !in_lo;
    if (a.include_mask && n < a.n && a.include_mask[n]) s = true;
    if (s) sel |= 1u << j;
  }

  uint32_t total;
  uint32_t pos = block_excl_scan((uint32_t)__popc(sel), tmp, total);
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
  }
  if (t == 0 && a.count_out) a.count_out[row] = (int32_t)total;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  const int need = (a.n + kSelThreads - 1) / kSelThreads;
  dim3 grid(a.rows), block(kSelThreads);
  if (need <= 1) hipLaunchKernelGGL(select_kernel<1>, grid, block, 0, s, a);
  else if (need <= 2) hipLaunchKernelGGL(select_kernel<2>, grid, block, 0, s, a);
  else if (need <= 4) hipLaunchKernelGGL(select_kernel<4>, grid, block, 0, s, a);
  else if (need <= 8) hipLaunchKernelGGL(select_kernel<8>, grid, block, 0, s, a);
  else if (need <= 16) hipLaunchKernelGGL(select_kernel<16>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(select_kernel<32>, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace sffn
