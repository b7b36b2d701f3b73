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
// streams either top rows (16-byte bf16 loads, 8 outputs per lane) or
// middle rows (4-byte code loads, 8 outputs per lane, so both tiers share
// the lane -> output mapping).  The middle tier is decoded in registers:
// x_j * What[j][o] = (x_j scale_js) q_jo + x_j zero_js, where the second term
// is the same for all outputs of the segment and is summed once per lane.
// Partials are summed in chunk order by the shared split-K reduction.
#include <hip/hip_fp16.h>

#include "sffn_splitk.h"

namespace sffn {

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)h));
}

struct SegBounds { int b[5]; };

__global__ __launch_bounds__(1024) void tiered_kernel(TierArgs a, int KS_top, int KS_mid,
                                                      float* partials) {
  __shared__ float4 red[kWaves][kTileCols / 4];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int col = tile * kTileCols + 8 * lane;
  const bool col_ok = col < a.d_out;

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;

  if (ks < KS_top) {
    int n = a.cnt_top ? *a.cnt_top : 0;
    n = n < a.k_top_max ? n : a.k_top_max;
    n = n > 0 ? n : 0;
    const int chunk = (n + KS_top - 1) / KS_top;
    const int k0 = ks * chunk, k1 = min(n, k0 + chunk);
    for (int kb = k0 + w; kb < k1; kb += kWaves * U) {
      float xv[U];
      uint4 wv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = kb + kWaves * u;
        const bool ok = it < k1;
        const int row = ok ? a.idx_top[it] : 0;
        xv[u] = ok ? a.x[row] : 0.f;
        wv[u] = (ok && col_ok) ? load_stream16(a.Wt + (size_t)row * a.ld_w + col)
                               : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[8];
        unpack8(wv[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(xv[u], f[e], acc[e]);
      }
    }
  } else {
    const int m = ks - KS_top;
    int n = a.cnt_mid ? *a.cnt_mid : 0;
    n = n < a.k_mid_max ? n : a.k_mid_max;
    n = n > 0 ? n : 0;
    const int chunk = (n + KS_mid - 1) / KS_mid;
    const int k0 = m * chunk, k1 = min(n, k0 + chunk);
    int seg = 0;
#pragma unroll
    for (int s = 1; s < 4; ++s)
      if (s < a.n_seg && col >= a.seg_bounds[s]) seg = s;
    const int hdr_off = 4 * seg;
    const int code_off = 16 + (col >> 1);
    float zacc = 0.f;
    for (int kb = k0 + w; kb < k1; kb += kWaves * U) {
      float xv[U];
      uint32_t hdr[U], codes[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int it = kb + kWaves * u;
        const bool ok = it < k1;
        const int row = ok ? a.idx_mid[it] : 0;
        const uint8_t* rec = a.rec + (size_t)row * a.rec_bytes;
        xv[u] = ok ? a.x[row] : 0.f;
        hdr[u] = ok ? *reinterpret_cast<const uint32_t*>(rec + hdr_off) : 0u;
        codes[u] = (ok && col_ok) ? load_stream4(rec + code_off) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float sc = half_bits_to_float(hdr[u] & 0xFFFFu);
        const float z = half_bits_to_float(hdr[u] >> 16);
        const float sx = xv[u] * sc;
        zacc = fmaf(xv[u], z, zacc);
        const uint32_t lo = codes[u] & 0x0F0F0F0Fu;
        const uint32_t hi = (codes[u] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          acc[2 * b] = fmaf(sx, (float)((lo >> (8 * b)) & 0xFFu), acc[2 * b]);
          acc[2 * b + 1] = fmaf(sx, (float)((hi >> (8 * b)) & 0xFFu), acc[2 * b + 1]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += zacc;
  }

  const float part = wg_reduce_cols(red, acc);
  const int c = tile * kTileCols + (int)threadIdx.x;
  if (threadIdx.x < kTileCols && c < a.d_out) partials[(size_t)ks * a.d_out + c] = part;
}

hipError_t launch_tiered(const TierArgs& a, hipStream_t s) {
  const int col_tiles = (a.d_out + kTileCols - 1) / kTileCols;
  // split the chunks between the tiers in proportion to the bytes each reads
  const double top_bytes = (double)a.k_top_max * a.d_out * 2.0;
  const double mid_bytes = (double)a.k_mid_max * (a.d_out / 2.0 + 4.0);
  int total = pick_split_b1((long)a.k_top_max + a.k_mid_max, col_tiles);
  if (total < 2) total = 2;
  int ks_top = (int)(total * top_bytes / (top_bytes + mid_bytes + 1e-30) + 0.5);
  if (a.k_top_max == 0) ks_top = 0;
  else if (ks_top < 1) ks_top = 1;
  int ks_mid = total - ks_top;
  if (a.k_mid_max == 0) ks_mid = 0;
  else if (ks_mid < 1) ks_mid = 1;
  if (ks_top + ks_mid == 0) ks_mid = 1;   // nothing to read: one chunk writes y
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes);
  hipLaunchKernelGGL(tiered_kernel, dim3(col_tiles, ks_top + ks_mid), dim3(1024), 0, s, a, ks_top,
                     ks_mid, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(partials, ks_top + ks_mid, 1, 1, a.d_out, nullptr, a.y, a.d_out,
                              a.accumulate, s);
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
