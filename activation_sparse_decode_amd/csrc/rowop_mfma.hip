// Activations for several tokens at once on MFMA (batched decode, and the
// dense prefill / calibration passes that feed the selection).
//
// C[m][n] = sum_k X[m][k] W[n][k]: tokens are the M dimension, neurons the
// N dimension.  Neuron-major weights are already K-contiguous, so each lane
// feeds its MFMA B operand with one 16-byte load of a weight row.  The fp32
// activations are split into bf16 hi + lo parts (x = hi + lo to ~2^-17
// relative) and contracted with two MFMAs into one fp32 accumulator, so the
// result keeps fp32-grade accuracy with bf16 weights.
//
// Work split: a workgroup owns a 16-neuron x 16-token tile; its four waves
// take disjoint quarters of K and are summed in LDS in a fixed order.
#include "sffn_device.h"

namespace sffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum { kOpGlu = 0, kOpDotRelu = 1, kOpGated = 2, kOpDot = 4 };

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Split 8 fp32 values into bf16 hi and lo parts (packed pairs, memory order).
__device__ __forceinline__ void split8(const float4& p, const float4& q, uint4& hi, uint4& lo) {
  const float v[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
  uint32_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = f32_to_bf16_rne(v[e]);
    const float r = v[e] - __uint_as_float(h[e] << 16);
    l[e] = f32_to_bf16_rne(r);
  }
  hi = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
  lo = make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16), l[6] | (l[7] << 16));
}

template <int OP>
__global__ __launch_bounds__(256) void rowop_mfma_kernel(RowOpArgs a) {
  __shared__ f32x4 red[2][4][64];
  __shared__ float sq_red[4][16];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nl = lane & 15;
  const int g = lane >> 4;
  const int m0 = blockIdx.y * 16;
  const int t0 = blockIdx.x * 16;

  int n_items;
  if (a.idx) {
    int c = *a.count;
    c = c < a.k_max ? c : a.k_max;
    n_items = (c > 0 ? c : 0) * a.group;
  } else {
    n_items = a.n_rows;
  }
  if (t0 >= n_items) return;  // uniform over the workgroup

  const int it = t0 + nl;
  const bool live = it < n_items;
  int row = 0;
  if (live) {
    if (a.idx) {
      const int q = it / a.group;
      row = a.idx[q] * a.group + (it - q * a.group);
    } else {
      row = it;
    }
  }
  const int tok = m0 + nl;
  const bool tok_ok = tok < a.batch;

  const uint16_t* w0p = a.W0 + (size_t)row * a.ld_w + g * 8;
  const uint16_t* w1p = a.W1 + (size_t)row * a.ld_w + g * 8;
  const float* xp = a.x + (size_t)(tok_ok ? tok : 0) * a.ld_in + g * 8;

  const int ksteps = a.d >> 5;
  const int ks0 = (ksteps * w) >> 2;
  const int ks1 = (ksteps * (w + 1)) >> 2;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};
  float sq = 0.f;
  const uint4 zero4 = make_uint4(0, 0, 0, 0);

  for (int ks = ks0; ks < ks1; ++ks) {
    const int k = ks * 32;
    uint4 wa = zero4, wb = zero4;
    if (OP != kOpGated) wa = live ? *reinterpret_cast<const uint4*>(w0p + k) : zero4;
    if (OP == kOpGlu || OP == kOpGated) wb = live ? *reinterpret_cast<const uint4*>(w1p + k) : zero4;
    float4 p = make_float4(0.f, 0.f, 0.f, 0.f), q = p;
    if (tok_ok) {
      p = *reinterpret_cast<const float4*>(xp + k);
      q = *reinterpret_cast<const float4*>(xp + k + 4);
    }
    {
      sq = fmaf(p.x, p.x, sq); sq = fmaf(p.y, p.y, sq); sq = fmaf(p.z, p.z, sq); sq = fmaf(p.w, p.w, sq);
      sq = fmaf(q.x, q.x, sq); sq = fmaf(q.y, q.y, sq); sq = fmaf(q.z, q.z, sq); sq = fmaf(q.w, q.w, sq);
    }
    uint4 xh, xl;
    split8(p, q, xh, xl);
    if (OP != kOpGated) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xh), as_bf16x8(wa), acc0, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xl), as_bf16x8(wa), acc0, 0, 0, 0);
    }
    if (OP == kOpGlu || OP == kOpGated) {
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xh), as_bf16x8(wb), acc1, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xl), as_bf16x8(wb), acc1, 0, 0, 0);
    }
  }

  red[0][w][lane] = acc0;
  red[1][w][lane] = acc1;
  {
    // lanes nl, nl+16, nl+32, nl+48 hold token nl's squares over this wave's K range
    sq += __shfl_xor(sq, 16, kWave);
    sq += __shfl_xor(sq, 32, kWave);
    if (g == 0) sq_red[w][nl] = sq;
  }
  __syncthreads();
  if (w != 0) return;

  f32x4 s0 = red[0][0][lane], s1 = red[1][0][lane];
#pragma unroll
  for (int ww = 1; ww < 4; ++ww) {
    const f32x4 t0v = red[0][ww][lane], t1v = red[1][ww][lane];
    s0 += t0v;
    s1 += t1v;
  }

  // C layout of the 16x16 MFMA: lane l, register i holds row m = 4*(l/16)+i
  // (token) and column n = l%16 (neuron).
  if (!live) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 4 * g + i;
    const int b = m0 + m;
    if (b >= a.batch) continue;
    // optional unit-gain RMSNorm of token b's input, applied to the dot products
    const float ss = sq_red[0][m] + sq_red[1][m] + sq_red[2][m] + sq_red[3][m];
    const float inv = a.rms_eps > 0.f ? 1.f / sqrtf(ss / (float)a.d + a.rms_eps) : 1.f;
    float v;
    if (OP == kOpGlu) {
      const float gg = s0[i] * inv;
      v = (gg / (1.f + expf(-gg))) * (s1[i] * inv);
    } else if (OP == kOpDotRelu) {
      v = fmaxf(s0[i] * inv - a.tau_scale * sqrtf(ss) * inv, 0.f);
    } else if (OP == kOpGated) {
      v = a.aux[(size_t)b * a.ld_aux + row] * (s1[i] * inv);
    } else {
      v = s0[i] * inv;
    }
    if (a.accumulate) v += a.out[(size_t)b * a.ld_out + row];
    a.out[(size_t)b * a.ld_out + row] = v;
    if (a.key_out) a.key_out[(size_t)b * a.ld_out + row] = key_abs(v);
  }
}

hipError_t launch_rowop_mfma(const RowOpArgs& a, hipStream_t s) {
  const long items = a.idx ? (long)a.k_max * a.group : (long)a.n_rows;
  const int nt = (int)((items + 15) / 16);
  const int mt = (a.batch + 15) / 16;
  if (nt == 0) return hipSuccess;
  dim3 grid(nt, mt);
  switch (a.op) {
    case kOpGlu: hipLaunchKernelGGL(rowop_mfma_kernel<kOpGlu>, grid, dim3(256), 0, s, a); break;
    case kOpDotRelu: hipLaunchKernelGGL(rowop_mfma_kernel<kOpDotRelu>, grid, dim3(256), 0, s, a); break;
    case kOpGated: hipLaunchKernelGGL(rowop_mfma_kernel<kOpGated>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(rowop_mfma_kernel<kOpDot>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace sffn
