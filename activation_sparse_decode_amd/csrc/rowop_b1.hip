// Row dot products at batch 1, streamed from HBM.
//
// out_n = f(W0[n].x, W1[n].x) for the processed rows n, with the magnitude
// key bits(|out_n|) written alongside (the ranking input of the selection
// step; SelectInfer §3 records |a| at the input of down_proj).  The same
// kernels run the down projection of a compacted neuron set (plain dot of
// each output row with the compacted activations, added to the residual).
// Skipped neurons are never read.  The optional RMSNorm of x scales the
// reduced dot products (W.(x s) = s (W.x)).
//
// Two ops serve the predictor-driven ReLU-sparse FFN (PowerInfer-2 guide,
// "Online Predictor"): PREDICT computes the cluster logits z = W x + b of
// the linear predictor and keys the clusters whose activation probability
// sigmoid(z) exceeds the threshold (the host passes the equivalent fp32
// logit threshold) so one selection compacts them; GLU_RELU computes the
// thresholded ReGLU max(W_g x - tau, 0) * (W_u x) of the predicted rows in
// one pass over both matrices.
//
// Rows up to 5120 wide (every shape of the workloads here) take the
// wave-per-row kernel: a wave owns whole rows, lane l the 16-byte chunks l,
// l+64, ... (NCH of them) of each, so one wave instruction reads 1 KiB of a
// row and the lane keeps the matching 8*NCH entries of x in registers.  A
// row's loads (both matrices for the GLU) are issued together, the dot
// product is reduced across the wave with DPP moves only, and lane 0 writes
// the result: no LDS, no barrier.  Measured on MI355X against the
// workgroup-per-row kernel below: 5-12% faster on every workload shape
// (e.g. 12.2 vs 13.9 us for 8192 SwiGLU neurons of 2048, 54 vs 60 us for
// 17408 of 5120).  Wider rows take the workgroup-per-row kernel: a
// workgroup spans one row, thread t owns chunks t, t+TPB, ... and the waves'
// partial sums meet in LDS.
#include "sffn_device.h"

namespace sffn {

enum { kOpGlu = 0, kOpDotRelu = 1, kOpGated = 2, kOpDot = 4, kOpGluRelu = 5, kOpPredict = 6,
       kOpDotReluC = 7 };

// Ops with the thresholded ReLU gate max(W x - tau, 0).
template <int OP>
constexpr bool relu_gate_op() { return OP == kOpDotRelu || OP == kOpDotReluC; }

// Key of a row-op value: the magnitude key, or for PREDICT the order-
// preserving key of a logit above the threshold (nonzero) and 0 otherwise.
template <int OP>
__device__ __forceinline__ uint32_t out_key(float v, float thr) {
  if (OP == kOpPredict) return v > thr ? key_signed(v) : 0u;
  return key_abs(v);
}

// Key output of one processed row: per row, or for DOT_RELU_CLUSTER the max
// of the magnitude keys of a cluster's nonzero rows, raised atomically in
// key_out[row / group] (a zero row leaves it as it is).
template <int OP>
__device__ __forceinline__ void store_key(uint32_t* key_out, int row, int group, float v, float thr) {
  if (OP == kOpDotReluC) {
    if (v > 0.f) atomicMax(key_out + row / group, key_abs(v));
  } else {
    key_out[row] = out_key<OP>(v, thr);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------ wave per row

constexpr int kWaveMaxChunks = 10;   // 16-byte chunks per lane: rows up to 5120 wide

// Wave gw of W handles the items gw + W*k, k < its (<= 64, guaranteed by the
// launch).  Lane k fetches the row of item k (and, when used, the value it
// adds to and its gate) once; the item loop reads them back with readlane.
// Every load is unconditional: chunks past the row end re-read chunk 0
// against x = 0.
template <int OP, int NCH>
__global__ __launch_bounds__(256) void rowop_wave_kernel(RowOpArgs a) {
  constexpr bool kUse0 = OP != kOpGated;
  constexpr bool kUse1 = OP == kOpGlu || OP == kOpGated || OP == kOpGluRelu;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (int)(blockDim.x >> 6) + wave_id();
  const int W = gridDim.x * (int)(blockDim.x >> 6);
  const int nchunk = a.d >> 3;

  int n_items;
  if (a.idx) {
    int c = *a.count;
    c = c < a.k_max ? c : a.k_max;
    n_items = (c > 0 ? c : 0) * a.group;
  } else {
    n_items = a.n_rows;
  }
  if (gw >= n_items) return;
  const int its = (n_items - gw + W - 1) / W;

  int lane_row;
  {
    const int it = gw + W * (lane < its ? lane : 0);
    if (a.idx) {
      const int q = it / a.group;
      lane_row = a.idx[q] * a.group + (it - q * a.group);
    } else {
      lane_row = it;
    }
  }
  float lane_pv, lane_av = 0.f;
  {
    const float* pp = a.accumulate ? a.out + lane_row : a.x;
    lane_pv = *pp;
    if (OP == kOpGated) lane_av = a.aux[lane_row];
    if (OP == kOpPredict) {   // bias, if any (the load is unconditional)
      const float b = *(a.aux ? a.aux + lane_row : a.x);
      lane_av = a.aux ? b : 0.f;
    }
  }

  // x is requested first but consumed only after the first row's weights
  // are requested (x is usually the previous kernel's output, so waiting for
  // it first would add a round trip to every wave); the empty asm (a
  // compiler barrier that also redefines `zero`) keeps the conversion of x
  // and the norm from moving ahead of those loads.  With one weight matrix
  // the row loads are double-buffered: row k+1 is requested before row k is
  // reduced, so the wave's reduction and store overlap the next row's
  // fetch (measured on 28 layers of 3072 x 2736 down projections: 5.31 ->
  // 5.11 us per launch).  With two matrices (gate and up) the registers go
  // to the second matrix instead (measured: no gain from a second buffer),
  // and the loop is rotated: reduce and store row k, then request row k+1.
  int coff[NCH];
  float xm[NCH];
  float4 xp[NCH], xq[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    coff[j] = c < nchunk ? 8 * c : 0;
    xm[j] = c < nchunk ? 1.f : 0.f;
    xp[j] = *reinterpret_cast<const float4*>(a.x + coff[j]);
    xq[j] = *reinterpret_cast<const float4*>(a.x + coff[j] + 4);
  }
  constexpr int NB = (kUse0 && kUse1) ? 1 : 2;   // row buffers
  uint4 v0[NB][NCH], v1[NB][NCH];
  auto fetch = [&](int r, int b) {
    const size_t base = (size_t)r * a.ld_w;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (kUse0) v0[b][j] = load_stream(a.W0 + base + coff[j]);
      if (kUse1) v1[b][j] = load_stream(a.W1 + base + coff[j]);
    }
  };
  auto row_of = [&](int k) { return a.idx ? __builtin_amdgcn_readlane(lane_row, k) : gw + W * k; };
  fetch(row_of(0), 0);

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
  float inv = 1.f, tau = 0.f;
  if (relu_gate_op<OP>() || OP == kOpGluRelu || a.rms_eps > 0.f) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(xr[j][e], xr[j][e], ss);
    ss = wave_sum(ss);
    if (a.rms_eps > 0.f) inv = 1.f / sqrtf(ss / (float)a.d + a.rms_eps);
    tau = a.tau_scale * sqrtf(ss) * inv;   // ||x s|| for the ReLU threshold
  }

  // reduce row k (held in buffer b) and store its result
  auto finish = [&](int k, int b) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float f[8];
      if (kUse0) {
        unpack8(v0[b][j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s0 = fmaf(f[e], xr[j][e], s0);
      }
      if (kUse1) {
        unpack8(v1[b][j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s1 = fmaf(f[e], xr[j][e], s1);
      }
    }
    if (kUse0) s0 = wave_sum(s0);
    if (kUse1) s1 = wave_sum(s1);
    const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_pv), k));
    const float av = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_av), k));
    const int r = row_of(k);
    if (lane == 0) {
      const float g = s0 * inv, u = s1 * inv;
      float v;
      if (OP == kOpGlu) {
        v = (g / (1.f + expf(-g))) * u;
      } else if (relu_gate_op<OP>()) {
        v = fmaxf(g - tau, 0.f);
      } else if (OP == kOpGated) {
        v = av * u;
      } else if (OP == kOpGluRelu) {
        v = fmaxf(g - tau, 0.f) * u;
      } else if (OP == kOpPredict) {
        v = g + av;
      } else {
        v = g;
      }
      if (a.accumulate) v += pv;
      a.out[r] = v;
      if (a.key_out) store_key<OP>(a.key_out, r, a.group, v, a.tau_scale);
    }
  };

  if constexpr (NB == 2) {
    for (int k = 0; k < its; k += 2) {
      if (k + 1 < its) fetch(row_of(k + 1), 1);
      finish(k, 0);
      if (k + 1 >= its) break;
      if (k + 2 < its) fetch(row_of(k + 2), 0);
      finish(k + 1, 1);
    }
  } else {
    for (int k = 0;;) {
      finish(k, 0);
      if (++k >= its) break;
      fetch(row_of(k), 0);
    }
  }
}

template <int OP, int NCH>
static hipError_t launch_wave(const RowOpArgs& a, hipStream_t s) {
  // Workgroups of four waves, a multiple of 256 of them (the same number on
  // every CU): 256 up to ~3000 rows, doubling per doubling of the rows up to
  // 2048; at most 64 rows per wave.  A gathered launch is sized by its bound
  // k_max while the device count is often a fraction of it (MoE clusters:
  // ~20%): it takes at most 512 (measured on 2 x ~90 of 448 clusters of
  // 14336 x 4096 experts: 10.7 us at 512 vs 13.7 us at 2048 workgroups).
  const long items = a.idx ? (long)a.k_max * a.group : (long)a.n_rows;
  long blocks = 256;
  while (blocks < 2048 && items >= 6 * blocks * 2) blocks *= 2;
  if (a.idx && blocks > 512) blocks = 512;
  if (blocks * 4 > items) blocks = (items + 3) / 4;
  if (blocks * 4 * 64 < items) blocks = (items + 255) / 256;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((rowop_wave_kernel<OP, NCH>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_wave_op(const RowOpArgs& a, hipStream_t s) {
  switch ((a.d / 8 + 63) / 64) {
    case 0:
    case 1: return launch_wave<OP, 1>(a, s);
    case 2: return launch_wave<OP, 2>(a, s);
    case 3: return launch_wave<OP, 3>(a, s);
    case 4: return launch_wave<OP, 4>(a, s);
    case 5: return launch_wave<OP, 5>(a, s);
    case 6: return launch_wave<OP, 6>(a, s);
    case 7:
    case 8: return launch_wave<OP, 8>(a, s);
    default: return launch_wave<OP, kWaveMaxChunks>(a, s);
  }
}

// ------------------------------------------------------------ several row lists

// 64-bit pointer held per lane, read back for lane k as a wave-uniform value.
template <typename T>
__device__ __forceinline__ T* lane_ptr(T* p, int k) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, k);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), k);
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// The wave-per-row kernel over the concatenated items of several lists (the
// routed experts of a MoE layer in one launch): lane k resolves item k's
// list and row once and keeps the row's weight and output addresses, which
// the item loop reads back with readlane.  Per row the arithmetic is the
// single-list kernel's, so each list's results are bitwise those of a
// separate call.
template <int OP, int NCH>
__global__ __launch_bounds__(256) void rowop_lists_kernel(RowOpListsArgs L) {
  constexpr bool kUse0 = OP != kOpGated;
  constexpr bool kUse1 = OP == kOpGlu || OP == kOpGated || OP == kOpGluRelu;
  const RowOpArgs& a = L.base;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (int)(blockDim.x >> 6) + wave_id();
  const int W = gridDim.x * (int)(blockDim.x >> 6);
  const int nchunk = a.d >> 3;

  // list l covers the items [pre[l], pre[l + 1])
  int pre[kMaxRowLists + 1];
  int n_items = 0;
#pragma unroll
  for (int l = 0; l < kMaxRowLists; ++l) {
    pre[l] = n_items;
    int c = 0;
    if (l < L.n) {
      if (L.idx[l]) {
        c = *L.count[l];
        c = c < L.k_max[l] ? c : L.k_max[l];
        c = (c > 0 ? c : 0) * a.group;
      } else {
        c = a.n_rows;
      }
    }
    n_items += c;
  }
  pre[kMaxRowLists] = n_items;
  if (gw >= n_items) return;
  const int its = (n_items - gw + W - 1) / W;

  const uint16_t* lp0;
  const uint16_t* lp1;
  float* lpo;
  uint32_t* lpk;
  float lane_pv, lane_av = 0.f;
  {
    const int it = gw + W * (lane < its ? lane : 0);
    int li = 0;
#pragma unroll
    for (int l = 1; l < kMaxRowLists; ++l) li += (l < L.n && it >= pre[l]) ? 1 : 0;
    const uint16_t* w0 = L.W0[0];
    const uint16_t* w1 = L.W1[0];
    const int32_t* ix = L.idx[0];
    const float* ax = L.aux[0];
    float* o = L.out[0];
    uint32_t* ko = L.key_out[0];
    int p = 0;
#pragma unroll
    for (int l = 1; l < kMaxRowLists; ++l) {
      if (li == l) {
        w0 = L.W0[l]; w1 = L.W1[l]; ix = L.idx[l]; ax = L.aux[l]; o = L.out[l]; ko = L.key_out[l];
        p = pre[l];
      }
    }
    const int q0 = it - p;
    int row;
    if (ix) {
      const int q = q0 / a.group;
      row = ix[q] * a.group + (q0 - q * a.group);
    } else {
      row = q0;
    }
    lp0 = w0 + (size_t)row * a.ld_w;
    lp1 = kUse1 ? w1 + (size_t)row * a.ld_w : lp0;
    lpo = o + row;
    lpk = ko ? ko + (OP == kOpDotReluC ? row / a.group : row) : nullptr;
    lane_pv = *(a.accumulate ? lpo : a.x);
    if (OP == kOpGated) lane_av = ax[row];
    if (OP == kOpPredict) {
      const float b = *(ax ? ax + row : a.x);
      lane_av = ax ? b : 0.f;
    }
  }

  int coff[NCH];
  float xm[NCH];
  float4 xp[NCH], xq[NCH];
#pragma unroll
  for (int j = 0; j < NCH; ++j) {
    const int c = lane + 64 * j;
    coff[j] = c < nchunk ? 8 * c : 0;
    xm[j] = c < nchunk ? 1.f : 0.f;
    xp[j] = *reinterpret_cast<const float4*>(a.x + coff[j]);
    xq[j] = *reinterpret_cast<const float4*>(a.x + coff[j] + 4);
  }
  constexpr int NB = (kUse0 && kUse1) ? 1 : 2;   // row buffers, as above
  uint4 v0[NB][NCH], v1[NB][NCH];
  auto fetch = [&](int k, int b) {
    const uint16_t* p0 = lane_ptr(lp0, k);
    const uint16_t* p1 = kUse1 ? lane_ptr(lp1, k) : p0;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      if (kUse0) v0[b][j] = load_stream(p0 + coff[j]);
      if (kUse1) v1[b][j] = load_stream(p1 + coff[j]);
    }
  };
  fetch(0, 0);

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
  float inv = 1.f, tau = 0.f;
  if (relu_gate_op<OP>() || OP == kOpGluRelu || a.rms_eps > 0.f) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(xr[j][e], xr[j][e], ss);
    ss = wave_sum(ss);
    if (a.rms_eps > 0.f) inv = 1.f / sqrtf(ss / (float)a.d + a.rms_eps);
    tau = a.tau_scale * sqrtf(ss) * inv;
  }

  auto finish = [&](int k, int b) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      float f[8];
      if (kUse0) {
        unpack8(v0[b][j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s0 = fmaf(f[e], xr[j][e], s0);
      }
      if (kUse1) {
        unpack8(v1[b][j], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s1 = fmaf(f[e], xr[j][e], s1);
      }
    }
    if (kUse0) s0 = wave_sum(s0);
    if (kUse1) s1 = wave_sum(s1);
    const float pv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_pv), k));
    const float av = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_av), k));
    float* po = lane_ptr(lpo, k);
    uint32_t* pk = lane_ptr(lpk, k);
    if (lane == 0) {
      const float g = s0 * inv, u = s1 * inv;
      float v;
      if (OP == kOpGlu) {
        v = (g / (1.f + expf(-g))) * u;
      } else if (relu_gate_op<OP>()) {
        v = fmaxf(g - tau, 0.f);
      } else if (OP == kOpGated) {
        v = av * u;
      } else if (OP == kOpGluRelu) {
        v = fmaxf(g - tau, 0.f) * u;
      } else if (OP == kOpPredict) {
        v = g + av;
      } else {
        v = g;
      }
      if (a.accumulate) v += pv;
      *po = v;
      if (pk) {
        if (OP == kOpDotReluC) {
          if (v > 0.f) atomicMax(pk, key_abs(v));
        } else {
          *pk = out_key<OP>(v, a.tau_scale);
        }
      }
    }
  };

  if constexpr (NB == 2) {
    for (int k = 0; k < its; k += 2) {
      if (k + 1 < its) fetch(k + 1, 1);
      finish(k, 0);
      if (k + 1 >= its) break;
      if (k + 2 < its) fetch(k + 2, 0);
      finish(k + 1, 1);
    }
  } else {
    for (int k = 0;;) {
      finish(k, 0);
      if (++k >= its) break;
      fetch(k, 0);
    }
  }
}

template <int OP, int NCH>
static hipError_t launch_lists_nch(const RowOpListsArgs& L, hipStream_t s) {
  long items = 0;
  for (int l = 0; l < L.n; ++l)
    items += L.idx[l] ? (long)L.k_max[l] * L.base.group : (long)L.base.n_rows;
  long blocks = 256;   // as launch_wave, gathered lists capped at 512
  while (blocks < 2048 && items >= 6 * blocks * 2) blocks *= 2;
  if (L.idx[0] && blocks > 512) blocks = 512;
  if (blocks * 4 > items) blocks = (items + 3) / 4;
  if (blocks * 4 * 64 < items) blocks = (items + 255) / 256;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((rowop_lists_kernel<OP, NCH>), dim3((unsigned)blocks), dim3(256), 0, s, L);
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_lists_op(const RowOpListsArgs& L, hipStream_t s) {
  switch ((L.base.d / 8 + 63) / 64) {
    case 0:
    case 1: return launch_lists_nch<OP, 1>(L, s);
    case 2: return launch_lists_nch<OP, 2>(L, s);
    case 3: return launch_lists_nch<OP, 3>(L, s);
    case 4: return launch_lists_nch<OP, 4>(L, s);
    case 5: return launch_lists_nch<OP, 5>(L, s);
    case 6: return launch_lists_nch<OP, 6>(L, s);
    case 7:
    case 8: return launch_lists_nch<OP, 8>(L, s);
    default: return launch_lists_nch<OP, kWaveMaxChunks>(L, s);
  }
}

hipError_t launch_rowop_lists(const RowOpListsArgs& L, hipStream_t s) {
  switch (L.base.op) {
    case kOpGlu: return launch_lists_op<kOpGlu>(L, s);
    case kOpDotRelu: return launch_lists_op<kOpDotRelu>(L, s);
    case kOpGated: return launch_lists_op<kOpGated>(L, s);
    case kOpGluRelu: return launch_lists_op<kOpGluRelu>(L, s);
    case kOpPredict: return launch_lists_op<kOpPredict>(L, s);
    case kOpDotReluC: return launch_lists_op<kOpDotReluC>(L, s);
    default: return launch_lists_op<kOpDot>(L, s);
  }
}

// ------------------------------------------------------------ workgroup per row

template <int OP, int CPT, int NPI>
__global__ __launch_bounds__(1024) void rowop_b1_kernel(RowOpArgs a) {
  constexpr bool kUse0 = OP != kOpGated;
  constexpr bool kUse1 = OP == kOpGlu || OP == kOpGated || OP == kOpGluRelu;
  constexpr int kVals = (kUse0 && kUse1) ? 2 : 1;   // dot products per row
  __shared__ float red[2][16][NPI * kVals];            // [parity][wave][row*vals]
  __shared__ float sq_red[16];

  const int t = threadIdx.x;
  const int lane = t & 63, w = wave_id();
  const int nw = blockDim.x >> 6;
  const int tpb = blockDim.x;
  const int nchunk = a.d >> 3;

  int n_items;
  if (a.idx) {
    int c = *a.count;
    c = c < a.k_max ? c : a.k_max;
    n_items = (c > 0 ? c : 0) * a.group;
  } else {
    n_items = a.n_rows;
  }

  // This thread's chunks of every row.  Chunks past the row end re-read the
  // row's first chunk (always valid) against x = 0, so every weight load is
  // unconditional: no branch around a load, nothing for the compiler to
  // wait on before the next one is issued.
  int coff[CPT];
  float xr[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = t + tpb * j;
    coff[j] = c < nchunk ? 8 * c : 0;
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

  // Rows of this workgroup: items base0 + i + stride * it.  With an index
  // list, one vector load per lane fetches the rows of the first 64 items
  // up front (lane l: iteration l / NPI, row l % NPI); later items, if any,
  // read their index when they are reached.
  const int stride = gridDim.x * NPI;
  const int base0 = blockIdx.x * NPI;
  int lane_row = 0;
  if (a.idx) {
    const int it = base0 + (lane / NPI) * stride + (lane % NPI);
    if (it < n_items) {
      const int q = it / a.group;
      lane_row = a.idx[q] * a.group + (it - q * a.group);
    }
  }
  auto row_of = [&](int k, int i) -> int {   // row of item base0 + i + stride * k (a live item)
    const int it = base0 + i + stride * k;
    if (!a.idx) return it;
    const int l = k * NPI + i;
    if (l < 64) return __builtin_amdgcn_readlane(lane_row, l);
    const int q = it / a.group;
    return a.idx[q] * a.group + (it - q * a.group);
  };

  const bool need_norm = relu_gate_op<OP>() || OP == kOpGluRelu || a.rms_eps > 0.f;
  bool have_norm = false;
  float tau = 0.f, inv = 1.f;
  int parity = 0;

  // Software pipeline: the weights of the next group of rows are requested
  // before the current group is reduced, so loads stay in flight across the
  // reductions and barriers and x is reused for the workgroup's whole life.
  int row[NPI];
  bool live[NPI];
  float prev[NPI];
  uint4 w0[NPI][CPT], w1[NPI][CPT];
  // With accumulate, the output value each row adds to is requested with the
  // row's weights, so the epilogue does not wait for it.
  auto fetch = [&](int k, int (&rw)[NPI], bool (&lv)[NPI], uint4 (&v0)[NPI][CPT],
                   uint4 (&v1)[NPI][CPT], float (&pv)[NPI]) {
#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      lv[i] = base0 + i + stride * k < n_items;
      rw[i] = lv[i] ? row_of(k, i) : rw[0];   // a dead row re-reads the group's first row
      pv[i] = a.accumulate ? a.out[rw[i]] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NPI; ++i)
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const size_t off = (size_t)rw[i] * a.ld_w + coff[j];
        if (kUse0) v0[i][j] = load_stream(a.W0 + off);
        if (kUse1) v1[i][j] = load_stream(a.W1 + off);
      }
  };
  int k = 0;
  if (base0 < n_items) fetch(0, row, live, w0, w1, prev);

  for (; base0 + stride * k < n_items; ++k) {
    int nrow[NPI];
    bool nlive[NPI];
    float nprev[NPI];
    uint4 n0[NPI][CPT], n1[NPI][CPT];
    const bool more = base0 + stride * (k + 1) < n_items;
    if (more) fetch(k + 1, nrow, nlive, n0, n1, nprev);

    if (need_norm && !have_norm) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(xr[j][e], xr[j][e], s);
      s = wave_sum(s);
      if (lane == 0) sq_red[w] = s;
    }

#pragma unroll
    for (int i = 0; i < NPI; ++i) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        float f[8];
        if (kUse0) {
          unpack8(w0[i][j], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) s0 = fmaf(f[e], xr[j][e], s0);
        }
        if (kUse1) {
          unpack8(w1[i][j], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) s1 = fmaf(f[e], xr[j][e], s1);
        }
      }
      if (kUse0) s0 = wave_sum(s0);
      if (kUse1) s1 = wave_sum(s1);
      if (lane == 0) {
        if (kUse0) red[parity][w][i * kVals] = s0;
        if (kUse1) red[parity][w][i * kVals + kVals - 1] = s1;
      }
    }
    __syncthreads();

    if (need_norm && !have_norm) {
      float s = 0.f;
      for (int ww = 0; ww < nw; ++ww) s += sq_red[ww];
      if (a.rms_eps > 0.f) inv = 1.f / sqrtf(s / (float)a.d + a.rms_eps);
      tau = a.tau_scale * sqrtf(s) * inv;   // ||x s|| for the ReLU threshold
      have_norm = true;
    }

    if (t < NPI && live[t < NPI ? t : 0]) {
      const int i = t;
      float g = 0.f, u = 0.f;
      for (int ww = 0; ww < nw; ++ww) {
        if (kUse0) g += red[parity][ww][i * kVals];
        if (kUse1) u += red[parity][ww][i * kVals + kVals - 1];
      }
      g *= inv;
      u *= inv;
      int r = 0;
      float pv = 0.f;
#pragma unroll
      for (int ii = 0; ii < NPI; ++ii) {
        r = (ii == i) ? row[ii] : r;
        pv = (ii == i) ? prev[ii] : pv;
      }
      float v;
      if (OP == kOpGlu) {
        v = (g / (1.f + expf(-g))) * u;
      } else if (relu_gate_op<OP>()) {
        v = fmaxf(g - tau, 0.f);
      } else if (OP == kOpGated) {
        v = a.aux[r] * u;
      } else if (OP == kOpGluRelu) {
        v = fmaxf(g - tau, 0.f) * u;
      } else if (OP == kOpPredict) {
        v = g + (a.aux ? a.aux[r] : 0.f);
      } else {
        v = g;
      }
      if (a.accumulate) v += pv;
      a.out[r] = v;
      if (a.key_out) store_key<OP>(a.key_out, r, a.group, v, a.tau_scale);
    }
    parity ^= 1;   // the next iteration writes the other LDS half
    if (more) {
#pragma unroll
      for (int i = 0; i < NPI; ++i) {
        row[i] = nrow[i];
        live[i] = nlive[i];
        prev[i] = nprev[i];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
          if (kUse0) w0[i][j] = n0[i][j];
          if (kUse1) w1[i][j] = n1[i][j];
        }
      }
    }
  }
}

template <int OP, int CPT, int NPI>
static hipError_t launch_cfg(const RowOpArgs& a, hipStream_t s, long cap) {
  const int nchunk = a.d >> 3;
  int tpb = (nchunk + CPT - 1) / CPT;
  tpb = (tpb + 63) / 64 * 64;
  const long items = a.idx ? (long)a.k_max * a.group : (long)a.n_rows;
  long blocks = (items + NPI - 1) / NPI;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((rowop_b1_kernel<OP, CPT, NPI>), dim3((unsigned)blocks), dim3(tpb), 0, s, a);
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_op(const RowOpArgs& a, hipStream_t s) {
  const int nchunk = a.d >> 3;
  if (nchunk <= 64 * kWaveMaxChunks) return launch_wave_op<OP>(a, s);
  // Measured on MI355X at the 28-layer stack shapes: two 16-byte chunks per
  // thread per row (128-320-thread workgroups), one row (GLU: one neuron)
  // per iteration, at most 1024 (GLU) / 2048 (single matrix) workgroups.
  const long cap = (OP == kOpGlu || OP == kOpGluRelu) ? 1024 : 2048;   // two matrices or one
  return launch_cfg<OP, 2, 1>(a, s, cap);    // nchunk <= 1024 (d <= 8192)
}

hipError_t launch_rowop_b1(const RowOpArgs& a, hipStream_t s) {
  switch (a.op) {
    case kOpGlu: return launch_op<kOpGlu>(a, s);
    case kOpDotRelu: return launch_op<kOpDotRelu>(a, s);
    case kOpGated: return launch_op<kOpGated>(a, s);
    case kOpGluRelu: return launch_op<kOpGluRelu>(a, s);
    case kOpPredict: return launch_op<kOpPredict>(a, s);
    case kOpDotReluC: return launch_op<kOpDotReluC>(a, s);
    default: return launch_op<kOpDot>(a, s);
  }
}

}  // namespace sffn
