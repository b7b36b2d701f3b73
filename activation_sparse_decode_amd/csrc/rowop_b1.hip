// Activations at batch 1: one row dot product per neuron, streamed from HBM.
//
// out_n = f(W0[n].x, W1[n].x) for the processed rows n, with the magnitude
// key bits(|out_n|) written alongside (the ranking input of the selection
// step; SelectInfer §3 records |a| at the input of down_proj).
//
// Layout: W rows are neuron-major bf16 (row n = neuron n's d input weights).
// A wave owns NPI neurons per iteration; lane l reads the 16-byte chunks
// l, l+64, l+128, ... of each row, so one wave instruction covers 1 KiB of a
// row, fully coalesced.  x is held in registers for the wave's lifetime
// (fp32, CPL chunks of 8 per lane) and every row is reduced across the wave
// with shuffles.  Skipped neurons are never read.
#include "sffn_device.h"

namespace sffn {

enum { kOpGlu = 0, kOpDotRelu = 1, kOpGated = 2 };

template <int OP, int CPL, int NPI>
__global__ __launch_bounds__(256) void rowop_b1_kernel(RowOpArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * 4;
  const int nchunk = a.d >> 3;

  int n_items;
  if (a.idx) {
    int c = *a.count;
    c = c < a.k_max ? c : a.k_max;
    n_items = (c > 0 ? c : 0) * a.group;
  } else {
    n_items = a.n_rows;
  }

  float xr[CPL][8];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
      const float4 p = *reinterpret_cast<const float4*>(a.x + 8 * c);
      const float4 q = *reinterpret_cast<const float4*>(a.x + 8 * c + 4);
      xr[j][0] = p.x; xr[j][1] = p.y; xr[j][2] = p.z; xr[j][3] = p.w;
      xr[j][4] = q.x; xr[j][5] = q.y; xr[j][6] = q.z; xr[j][7] = q.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xr[j][e] = 0.f;
    }
  }

  // Optional unit-gain RMSNorm of the input, applied to the dot products
  // (W.(x s) = s (W.x)); tau is taken on the normalised input.
  float tau = 0.f, inv = 1.f;
  if (OP == kOpDotRelu || a.rms_eps > 0.f) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(xr[j][e], xr[j][e], s);
    s = wave_sum(s);
    if (a.rms_eps > 0.f) inv = 1.f / sqrtf(s / (float)a.d + a.rms_eps);
    tau = a.tau_scale * sqrtf(s) * inv;
  }

  for (int base = wave * NPI; base < n_items; base += nwaves * NPI) {
    int row[NPI];
    bool live[NPI];
#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      const int it = base + i;
      live[i] = it < n_items;
      if (!live[i]) {
        row[i] = 0;
      } else if (a.idx) {
        const int q = it / a.group;
        row[i] = a.idx[q] * a.group + (it - q * a.group);
      } else {
        row[i] = it;
      }
    }

    uint4 w0[NPI][CPL], w1[NPI][CPL];
#pragma unroll
    for (int i = 0; i < NPI; ++i)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        const bool ok = live[i] && c < nchunk;
        const size_t off = (size_t)row[i] * a.ld_w + 8 * c;
        if (OP != kOpGated)
          w0[i][j] = ok ? *reinterpret_cast<const uint4*>(a.W0 + off) : make_uint4(0, 0, 0, 0);
        if (OP != kOpDotRelu)
          w1[i][j] = ok ? *reinterpret_cast<const uint4*>(a.W1 + off) : make_uint4(0, 0, 0, 0);
      }

    float acc0[NPI], acc1[NPI];
#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        float f[8];
        if (OP != kOpGated) {
          unpack8(w0[i][j], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) s0 = fmaf(f[e], xr[j][e], s0);
        }
        if (OP != kOpDotRelu) {
          unpack8(w1[i][j], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) s1 = fmaf(f[e], xr[j][e], s1);
        }
      }
      acc0[i] = (OP != kOpGated) ? wave_sum(s0) * inv : 0.f;
      acc1[i] = (OP != kOpDotRelu) ? wave_sum(s1) * inv : 0.f;
    }

#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      if (lane == i && live[i]) {
        float v;
        if (OP == kOpGlu) {
          const float g = acc0[i];
          v = (g / (1.f + expf(-g))) * acc1[i];
        } else if (OP == kOpDotRelu) {
          v = fmaxf(acc0[i] - tau, 0.f);
        } else {
          v = a.aux[row[i]] * acc1[i];
        }
        a.out[row[i]] = v;
        if (a.key_out) a.key_out[row[i]] = key_abs(v);
      }
    }
  }
}

template <int OP, int CPL>
static hipError_t launch_cpl(const RowOpArgs& a, hipStream_t s) {
  // Neurons per wave iteration: enough 16-byte loads in flight per lane
  // without spilling (two matrices for GLU).
  constexpr int NPI = (OP == kOpGlu) ? (CPL <= 6 ? 2 : 1) : (CPL <= 6 ? 4 : 2);
  const long items = a.idx ? (long)a.k_max * a.group : (long)a.n_rows;
  long waves = (items + NPI - 1) / NPI;
  if (waves > 4096) waves = 4096;
  if (waves < 1) waves = 1;
  const int blocks = (int)((waves + 3) / 4);
  hipLaunchKernelGGL((rowop_b1_kernel<OP, CPL, NPI>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_op(const RowOpArgs& a, hipStream_t s) {
  const int need = ((a.d >> 3) + 63) / 64;
  if (need <= 4) return launch_cpl<OP, 4>(a, s);
  if (need <= 6) return launch_cpl<OP, 6>(a, s);
  if (need <= 8) return launch_cpl<OP, 8>(a, s);
  if (need <= 10) return launch_cpl<OP, 10>(a, s);
  if (need <= 12) return launch_cpl<OP, 12>(a, s);
  return launch_cpl<OP, 16>(a, s);
}

hipError_t launch_rowop_b1(const RowOpArgs& a, hipStream_t s) {
  switch (a.op) {
    case kOpGlu: return launch_op<kOpGlu>(a, s);
    case kOpDotRelu: return launch_op<kOpDotRelu>(a, s);
    default: return launch_op<kOpGated>(a, s);
  }
}

}  // namespace sffn
