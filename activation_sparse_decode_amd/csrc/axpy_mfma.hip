// Gathered down projection for a batch of tokens on MFMA:
//   Y[b][o] = (acc ? Y[b][o] : 0) + alpha_b * sum_{i in U} m_bi a_b,i W^T[i][o]
// The union U of the tokens' selections is read once and contracted as one
// dense [batch x |U|] x [|U| x d] block; a token's masked-out neurons get an
// exact zero in the packed activation block, so they contribute nothing to
// that token (LeanStream "Permutation-Invariant Execution": a compacted
// neuron subset is an ordinary dense matrix).
//
// Step 1 (pack): A[m][k] = m_{m,row_k} a_{m,row_k}, split into bf16 hi + lo,
//   [Mpad][Kpad] each, zero beyond the batch and the row count.
// Step 2 (contract): tokens are the MFMA M dimension, output columns the N
//   dimension and gathered rows the K dimension.  W^T rows are contiguous
//   along N, so a workgroup stages a 64-row x 256-column tile in LDS with
//   16-byte coalesced loads, and each lane gathers its B operand (8 rows of
//   one column) from LDS.  The LDS row pitch (129 dwords) puts the four
//   K-groups of a wave on disjoint banks.  Split-K over row chunks; a second
//   kernel sums the chunks' partials in chunk order.
#include "sffn_splitk.h"

namespace sffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kOT = 256;          // output columns per workgroup
constexpr int kKT = 64;           // gathered rows per LDS stage
constexpr int kPitch = 258;       // LDS row pitch in bf16 elements (129 dwords)

__global__ __launch_bounds__(256) void pack_acts_kernel(AxpyArgs a, int Kpad, uint16_t* hi,
                                                        uint16_t* lo) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  const int m = blockIdx.y;
  if (k >= Kpad) return;
  const int n_items = item_count(a.idx, a.count, a.k_max, a.group, a.n_rows);
  float v = 0.f;
  if (m < a.batch && k < n_items) {
    const int row = item_row(a.idx, a.group, k);
    v = a.in[(size_t)m * a.ld_in + row];
    if (a.row_mask && !a.row_mask[(size_t)m * a.ld_mask + row]) v = 0.f;
  }
  const uint32_t h = f32_to_bf16_rne(v);
  const uint32_t l = f32_to_bf16_rne(v - __uint_as_float(h << 16));
  hi[(size_t)m * Kpad + k] = (uint16_t)h;
  lo[(size_t)m * Kpad + k] = (uint16_t)l;
}

__global__ __launch_bounds__(256) void axpy_mfma_kernel(AxpyArgs a, int KS, int Mpad, int Kpad,
                                                        const uint16_t* __restrict__ Ahi,
                                                        const uint16_t* __restrict__ Alo,
                                                        float* partials) {
  __shared__ uint32_t T[kKT * kPitch / 2];

  const int t = threadIdx.x;
  const int lane = t & 63, w = wave_id();
  const int nl = lane & 15, g = lane >> 4;
  const int ct = blockIdx.x, ks = blockIdx.y, mt = blockIdx.z;
  const int col0 = ct * kOT;
  const int m0 = mt * 16;

  const int n_items = item_count(a.idx, a.count, a.k_max, a.group, a.n_rows);
  int chunk = (n_items + KS - 1) / KS;
  chunk = (chunk + kKT - 1) / kKT * kKT;
  const int k0 = ks * chunk;
  const int k1 = min(n_items, k0 + chunk);
  const int nst = k1 > k0 ? (k1 - k0 + kKT - 1) / kKT : 0;

  // loader mapping: column chunk c (8 columns), rows r0 + 8j
  const int lc = t & 31;
  const int lr = t >> 5;
  const int lcol = col0 + 8 * lc;
  const bool lcol_ok = lcol < a.d;

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const uint16_t* Ahi_row = Ahi + (size_t)(m0 + nl) * Kpad + 8 * g;
  const uint16_t* Alo_row = Alo + (size_t)(m0 + nl) * Kpad + 8 * g;
  const uint16_t* Ts = reinterpret_cast<const uint16_t*>(T);

  for (int st = 0; st < nst; ++st) {
    const int kb = k0 + st * kKT;
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int it = kb + lr + 8 * j;
      const bool ok = it < k1 && lcol_ok;
      const int row = ok ? item_row(a.idx, a.group, it) : 0;
      v[j] = ok ? load_stream16(a.W + (size_t)row * a.ld_w + lcol)
                : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t* dst = T + ((lr + 8 * j) * kPitch + 8 * lc) / 2;
      dst[0] = v[j].x; dst[1] = v[j].y; dst[2] = v[j].z; dst[3] = v[j].w;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int kk = kb + 32 * s;
      const uint4 ah = *reinterpret_cast<const uint4*>(Ahi_row + kk);
      const uint4 al = *reinterpret_cast<const uint4*>(Alo_row + kk);
      const bf16x8 Ah = __builtin_bit_cast(bf16x8, ah);
      const bf16x8 Al = __builtin_bit_cast(bf16x8, al);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int o = 64 * w + 16 * nt + nl;
        const uint16_t* src = Ts + (32 * s + 8 * g) * kPitch + o;
        uint32_t b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b[j] = (uint32_t)src[(2 * j) * kPitch] | ((uint32_t)src[(2 * j + 1) * kPitch] << 16);
        const bf16x8 B = __builtin_bit_cast(bf16x8, make_uint4(b[0], b[1], b[2], b[3]));
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, B, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, B, acc[nt], 0, 0, 0);
      }
    }
  }

  // C layout: lane l, register i -> token m = 4*(l/16)+i, column n = l%16.
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int o = col0 + 64 * w + 16 * nt + nl;
    if (o < a.d) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        partials[((size_t)ks * Mpad + m0 + 4 * g + i) * a.d + o] = acc[nt][i];
    }
  }
}

int max_split_mfma(int mtiles) {
  const int k = 64 / mtiles;
  return k < 1 ? 1 : k;
}

hipError_t launch_axpy_mfma(const AxpyArgs& a, hipStream_t s) {
  const int Mt = (a.batch + 15) / 16;
  const int Mpad = Mt * 16;
  const long items = a.idx ? (long)a.k_max * a.group : (long)a.n_rows;
  const int Kpad = (int)((items + 63) / 64 * 64);
  const int col_tiles = (a.d + kOT - 1) / kOT;
  long KS = (768 + (long)col_tiles * Mt - 1) / ((long)col_tiles * Mt);
  const long by_rows = (items + kKT - 1) / kKT;
  if (KS > by_rows) KS = by_rows;
  if (KS > max_split_mfma(Mt)) KS = max_split_mfma(Mt);
  if (KS < 1) KS = 1;

  char* ws = reinterpret_cast<char*>(a.ws);
  float* partials = reinterpret_cast<float*>(ws + kWsHeaderBytes);
  const size_t part_bytes = align256((size_t)max_split_mfma(Mt) * Mpad * a.d * sizeof(float));
  uint16_t* hi = reinterpret_cast<uint16_t*>(ws + kWsHeaderBytes + part_bytes);
  uint16_t* lo = hi + align256((size_t)Mpad * Kpad * 2) / 2;

  if (Kpad > 0) {
    hipLaunchKernelGGL(pack_acts_kernel, dim3((Kpad + 255) / 256, Mpad), dim3(256), 0, s, a,
                       Kpad, hi, lo);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(axpy_mfma_kernel, dim3(col_tiles, (int)KS, Mt), dim3(256), 0, s, a, (int)KS,
                     Mpad, Kpad, hi, lo, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(partials, (int)KS, a.batch, Mpad, a.d, a.alpha, a.out, a.ld_out,
                              a.accumulate, s);
}

}  // namespace sffn
