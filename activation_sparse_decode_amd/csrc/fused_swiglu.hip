// Fused sparse-SwiGLU decode at batch 1: one pass per neuron of a set U
// forms the neuron's whole contribution to the FFN output,
//   a_n = silu(W_g[n].x) * (W_u[n].x),   y += a_n * W_down^T[n],
// reading the neuron's gate, up and down rows together (SelectInfer §5
// computes only the neurons of U; LeanStream "Permutation-Invariant
// Execution": the FFN output is a sum over hidden neurons, so each neuron
// can be finished on its own and the neurons taken in any order).
//
// A wave owns the neurons gw, gw + NW, ... (NW waves in the grid).  Lane l
// holds x at its 16-byte chunks c = l + 64 j (the wave-per-row layout: one
// wave instruction reads 1 KiB of a row) and a register copy of y at the
// same chunks.  Per neuron the gate, up and down loads are issued together;
// the two dot products are reduced across the wave with DPP moves, and
// every lane adds a_n times its chunks of the down row to its y.  The
// waves of a workgroup are summed in LDS in a fixed tree, the workgroup's
// partial y goes to the workspace, and the ordered split-K reduction adds
// the partials in workgroup order (and the value accumulated onto), so the
// result is reproducible run to run.  With the three rows of a neuron
// stored side by side (one record per neuron of a compacted U) the layer
// is a single sequential stream.
#include "sffn_splitk.h"

namespace sffn {

constexpr int kFusedWaves = 8;                    // waves per workgroup
constexpr int kFusedThreads = kFusedWaves * kWave;

template <int NCH>
__global__ __launch_bounds__(kFusedThreads) void fused_swiglu_kernel(FusedArgs a, float* partials) {
  extern __shared__ float4 red[];   // [kFusedWaves / 2][NCH][64][2]
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int gw = blockIdx.x * kFusedWaves + w;
  const int NW = gridDim.x * kFusedWaves;
  const int nchunk = a.d >> 3;

  int n_items;
  if (a.idx) {
    int c = *a.count;
    c = c < a.k_max ? c : a.k_max;
    n_items = c > 0 ? c : 0;
  } else {
    n_items = a.n_rows;
  }
  const int its = gw < n_items ? (n_items - gw + NW - 1) / NW : 0;

  int coff[NCH];
  float xm[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    coff[j] = c < nchunk ? 8 * c : 0;   // chunks past the row end re-read chunk 0 against x = 0
    xm[j] = c < nchunk ? 1.f : 0.f;
  }
  float y[NCH][8];
#pragma unroll
  for (int j = 0; j < NCH; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) y[j][e] = 0.f;

  if (its > 0) {
    // rows of this wave's first 64 neurons, one per lane, read back with readlane
    auto lane_row_of = [&](int ub) {
      const int it = gw + NW * (ub + lane < its ? ub + lane : ub);
      return a.idx ? a.idx[it] : it;
    };
    int lane_row = lane_row_of(0);
    // Rows wider than 3072 request the down row only once the gate and up
    // rows are consumed (their registers are free then; otherwise the
    // register copies of x and y leave no room for all three rows).
    constexpr bool kLateDown = NCH > 6;
    uint4 g[NCH], u[NCH], dn[NCH];
    auto fetch_down = [&](int r) {
      const size_t base = (size_t)r * a.ld_w;
#pragma unroll
      for (int j = 0; j < NCH; ++j) dn[j] = load_stream16(a.Wd + base + coff[j]);
    };
    auto fetch = [&](int r) {
      const size_t base = (size_t)r * a.ld_w;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        g[j] = load_stream16(a.Wg + base + coff[j]);
        u[j] = load_stream16(a.Wu + base + coff[j]);
        if (!kLateDown) dn[j] = load_stream16(a.Wd + base + coff[j]);
      }
    };
    fetch(__builtin_amdgcn_readlane(lane_row, 0));

    // x is consumed only after the first neuron's rows were requested (the
    // empty asm keeps its conversion and the norm behind those loads)
    float4 xp[NCH], xq[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      xp[j] = *reinterpret_cast<const float4*>(a.x + coff[j]);
      xq[j] = *reinterpret_cast<const float4*>(a.x + coff[j] + 4);
    }
    int zero = 0;
    asm volatile("" : "+v"(zero) : : "memory");
    const float zf = (float)zero;
    float xr[NCH][8];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const float m = xm[j] + zf;
      xr[j][0] = xp[j].x * m; xr[j][1] = xp[j].y * m;
      xr[j][2] = xp[j].z * m; xr[j][3] = xp[j].w * m;
      xr[j][4] = xq[j].x * m; xr[j][5] = xq[j].y * m;
      xr[j][6] = xq[j].z * m; xr[j][7] = xq[j].w * m;
    }
    float inv = 1.f;
    if (a.rms_eps > 0.f) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(xr[j][e], xr[j][e], ss);
      ss = wave_sum(ss);
      inv = 1.f / sqrtf(ss / (float)a.d + a.rms_eps);
    }

    for (int k = 0;;) {
      const int kk = k & 63;
      const int r = __builtin_amdgcn_readlane(lane_row, kk);
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        float f[8];
        unpack8(g[j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s0 = fmaf(f[e], xr[j][e], s0);
        unpack8(u[j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s1 = fmaf(f[e], xr[j][e], s1);
      }
      if (kLateDown) fetch_down(r);
      s0 = wave_sum(s0);
      s1 = wave_sum(s1);
      const float gg = s0 * inv, uu = s1 * inv;
      const float an = (gg / (1.f + expf(-gg))) * uu;
      if (a.a_out && lane == 0) a.a_out[r] = an;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        float f[8];
        unpack8(dn[j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[j][e] = fmaf(an, f[e], y[j][e]);
      }
      if (++k >= its) break;
      if ((k & 63) == 0) lane_row = lane_row_of(k);
      fetch(__builtin_amdgcn_readlane(lane_row, k & 63));
    }
  }

  // waves summed in a fixed tree: (w, w + 4), then (w, w + 2), then (0, 1)
#pragma unroll
  for (int half = kFusedWaves / 2; half >= 1; half >>= 1) {
    if (w >= half && w < 2 * half) {
      float4* dst = red + (size_t)(w - half) * NCH * 128;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        dst[(j * 64 + lane) * 2] = make_float4(y[j][0], y[j][1], y[j][2], y[j][3]);
        dst[(j * 64 + lane) * 2 + 1] = make_float4(y[j][4], y[j][5], y[j][6], y[j][7]);
      }
    }
    __syncthreads();
    if (w < half) {
      const float4* src = red + (size_t)w * NCH * 128;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const float4 p = src[(j * 64 + lane) * 2], q = src[(j * 64 + lane) * 2 + 1];
        y[j][0] += p.x; y[j][1] += p.y; y[j][2] += p.z; y[j][3] += p.w;
        y[j][4] += q.x; y[j][5] += q.y; y[j][6] += q.z; y[j][7] += q.w;
      }
    }
    __syncthreads();
  }
  if (w != 0) return;
  float* prow = partials + (size_t)blockIdx.x * a.d;
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    if (c < nchunk) {
      *reinterpret_cast<float4*>(prow + 8 * c) = make_float4(y[j][0], y[j][1], y[j][2], y[j][3]);
      *reinterpret_cast<float4*>(prow + 8 * c + 4) = make_float4(y[j][4], y[j][5], y[j][6], y[j][7]);
    }
  }
}

template <int NCH>
static hipError_t launch_fused_nch(const FusedArgs& a, int G, float* partials, hipStream_t s) {
  const size_t lds = (size_t)(kFusedWaves / 2) * NCH * 64 * 2 * sizeof(float4);
  hipLaunchKernelGGL(fused_swiglu_kernel<NCH>, dim3(G), dim3(kFusedThreads), lds, s, a, partials);
  return hipGetLastError();
}

hipError_t launch_fused_swiglu(const FusedArgs& a, hipStream_t s) {
  // one workgroup per CU at most (the register copies of x and y take a
  // wave's registers), never more than the ordered reduction adds
  const long items = a.idx ? (long)a.k_max : (long)a.n_rows;
  long G = (items + kFusedWaves - 1) / kFusedWaves;
  if (G > kMaxSplit) G = kMaxSplit;
  if (G < 1) G = 1;
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes);
  hipError_t e;
  switch ((a.d / 8 + 63) / 64) {
    case 0:
    case 1: e = launch_fused_nch<1>(a, (int)G, partials, s); break;
    case 2: e = launch_fused_nch<2>(a, (int)G, partials, s); break;
    case 3: e = launch_fused_nch<3>(a, (int)G, partials, s); break;
    case 4: e = launch_fused_nch<4>(a, (int)G, partials, s); break;
    case 5: e = launch_fused_nch<5>(a, (int)G, partials, s); break;
    case 6: e = launch_fused_nch<6>(a, (int)G, partials, s); break;
    default: e = launch_fused_nch<8>(a, (int)G, partials, s); break;
  }
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(partials, (int)G, 1, 1, a.d, nullptr, a.y, a.d, a.accumulate, s);
}

}  // namespace sffn
