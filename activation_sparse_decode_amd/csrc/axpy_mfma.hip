// Gathered down projection for a batch of tokens on MFMA:
//   Y[b][o] = (acc ? Y[b][o] : 0) + alpha_b * sum_{i in U} m_bi a_b,i W^T[i][o]
// The union U of the tokens' selections is read once and contracted as one
// dense [batch x |U|] x [|U| x d] block; a token's masked-out neurons get an
// exact zero in the packed activation block, so they contribute nothing to
// that token (LeanStream "Permutation-Invariant Execution": a compacted
// neuron subset is an ordinary dense matrix).
//
// Tokens are the MFMA M dimension, output columns the N dimension and
// gathered rows the K dimension.  W^T rows are contiguous along N, so a
// workgroup stages a 32-row x 256-column tile in LDS with 16-byte coalesced
// loads and each lane gathers its B operand (8 rows of one column) from
// LDS; the LDS row pitch (129 dwords) puts the four K-groups of a wave on
// disjoint banks.  The A operand is built per stage in the same kernel: the
// 16 tokens' activations of the stage's 64 rows are gathered (masked per
// token), split into bf16 hi + lo (x = hi + lo to ~2^-17 relative) and
// staged in LDS; two MFMAs (hi, lo) into one fp32 accumulator keep fp32-grade
// accuracy with bf16 weights.
//
// Pipeline: the chunk's row indices are read once into LDS; each stage's
// weights and activations are requested right after the previous stage was
// copied to LDS, so they are in flight while that stage is contracted.
// Split-K over row chunks; a second kernel sums the chunks' partials in
// chunk order.
//
// Without an index list and with mask_rows set, the union is formed here:
// a chunk is a range of neurons, and of each segment of it only the
// neurons whose mask is set for some token of the workgroup's token tile
// are listed (OR of the tokens' 16-byte mask words, then an in-order
// compaction), so exactly those rows are read, once, in index order.
#include "sffn_splitk.h"

namespace sffn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kOT = 256;          // output columns per workgroup
// Gathered rows per LDS stage.  32 (16 KB of weights per workgroup in
// flight) measured faster than 64 on the 17408 x 5120 union: batch 16 46.0
// -> 41.9 us, batch 8 -> 39.6, batch 4 39.1 -> 35.0 us with 512 workgroups
// (256 or 1024 workgroups slower).
constexpr int kKT = 32;
constexpr int kWJ = kKT / 8;         // weight loads per thread per stage
constexpr int kAR = kKT / 16;        // activations per thread per stage
constexpr int kPitch = 258;       // LDS row pitch in bf16 elements (129 dwords)
constexpr int kSeg = 2048;        // row indices held in LDS at a time
constexpr int kAPitch = kKT / 8 + 1;   // activation tile pitch in 16-byte units

__global__ __launch_bounds__(256) void axpy_mfma_kernel(AxpyArgs a, int KS, int Mpad,
                                                        float* partials) {
  __shared__ uint32_t T[kKT * kPitch / 2];
  __shared__ uint4 As[2][16][kAPitch];      // activations of the stage, bf16 hi / lo
  __shared__ int rows_s[kSeg];
  __shared__ uint32_t live_w[kSeg / 4];     // mask_rows: liveness byte per candidate
  __shared__ uint32_t cnt_w[4];             // mask_rows: live rows per wave

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

  // weight loader: column chunk lc (8 columns), rows lr + 8j.  Row-major: row
  // r at r * ld_w.  Packed column panels: the 256 columns of this workgroup's
  // tile are one contiguous 512-byte piece per row, rows back to back.
  const int lc = t & 31, lr = t >> 5;
  const int lcol = col0 + 8 * lc;
  const int lcolc = lcol < a.d ? lcol : 0;   // lanes past the last column re-read column 0
  const uint16_t* wbase = a.packed ? a.W + (size_t)ct * a.n_rows * kOT + 8 * lc : a.W + lcolc;
  const size_t wstride = a.packed ? (size_t)kOT : (size_t)a.ld_w;
  // activation loader: token am, rows kAR ar .. kAR ar + kAR - 1 of the stage
  const int am = t >> 4, ar = t & 15;
  const int tok = m0 + am;
  const bool tok_ok = tok < a.batch;
  const int tokc = tok_ok ? tok : 0;

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const uint16_t* Ts = reinterpret_cast<const uint16_t*>(T);

  for (int s0 = k0; s0 < k1; s0 += kSeg) {
    const int s1 = min(k1, s0 + kSeg);
    int nseg = s1 - s0;   // rows of this segment (mask_rows: its live rows)
    __syncthreads();   // the previous segment's readers of rows_s are done
    if (a.mask_rows) {
      // liveness: thread t ORs the 16-byte mask words of candidates
      // 16 (t & 127) .. +16 over tokens m0 + 8 (t >> 7) .. +8 of the tile
      for (int i = t; i < kSeg / 4; i += 256) live_w[i] = 0u;
      __syncthreads();
      {
        const int cb = t & 127, th = t >> 7;
        if (16 * cb < nseg) {
          uint4 o = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int b = m0 + 8 * th + e;
            if (b < a.batch) {
              const uint4 m = *reinterpret_cast<const uint4*>(a.row_mask + (size_t)b * a.ld_mask +
                                                             s0 + 16 * cb);
              o.x |= m.x; o.y |= m.y; o.z |= m.z; o.w |= m.w;
            }
          }
          atomicOr(&live_w[4 * cb], o.x);
          atomicOr(&live_w[4 * cb + 1], o.y);
          atomicOr(&live_w[4 * cb + 2], o.z);
          atomicOr(&live_w[4 * cb + 3], o.w);
        }
      }
      __syncthreads();
      // in-order compaction: thread t takes candidates 8t .. 8t + 7
      const uint32_t lw0 = live_w[2 * t], lw1 = live_w[2 * t + 1];
      uint32_t f = 0;   // bit k: candidate 8t + k is live
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint32_t byte = ((k < 4 ? lw0 : lw1) >> (8 * (k & 3))) & 0xFFu;
        f |= ((byte != 0u) && (8 * t + k < nseg) ? 1u : 0u) << k;
      }
      const uint32_t c = (uint32_t)__popc(f);
      uint32_t incl = c;   // inclusive scan of the counts over the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, off, kWave);
        if (lane >= off) incl += y;
      }
      if (lane == 63) cnt_w[w] = incl;
      __syncthreads();
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        before += ww < w ? cnt_w[ww] : 0u;
        total += cnt_w[ww];
      }
      uint32_t pos = before + incl - c;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if ((f >> k) & 1u) rows_s[pos++] = s0 + 8 * t + k;
      nseg = (int)total;
      if (nseg == 0) continue;   // uniform: no live row in this segment
      __syncthreads();
      // rows past the last live one repeat it (a live row; weight 0)
      const int nst = (nseg + kKT - 1) / kKT;
      const int last = rows_s[nseg - 1];
      __syncthreads();
      for (int i = nseg + t; i < nst * kKT; i += 256) rows_s[i] = last;
    } else {
      const int nst = (nseg + kKT - 1) / kKT;
      // rows past the segment end repeat its last row (a valid row; weight 0)
      for (int i = t; i < nst * kKT; i += 256)
        rows_s[i] = item_row(a.idx, a.group, min(s0 + i, s1 - 1));
    }
    const int nst = (nseg + kKT - 1) / kKT;
    __syncthreads();

    // raw loads only (no branch on a loaded value), so a stage's requests
    // stay in flight until the stage is copied to LDS
    const bool has_mask = a.row_mask != nullptr;
    const uint8_t* mrow = has_mask ? a.row_mask + (size_t)tokc * a.ld_mask
                                   : reinterpret_cast<const uint8_t*>(a.in);   // unused bytes
    uint4 v[kWJ];
    float xr[kAR];
    uint32_t mb[kAR];
    auto issue = [&](int st) {
      const int base = st * kKT;
#pragma unroll
      for (int j = 0; j < kWJ; ++j)
        v[j] = load_stream16(wbase + (size_t)rows_s[base + lr + 8 * j] * wstride);
#pragma unroll
      for (int e = 0; e < kAR; ++e) {
        const int r = rows_s[base + kAR * ar + e];
        xr[e] = a.in[(size_t)tokc * a.ld_in + r];
        mb[e] = mrow[r];
      }
    };
    issue(0);
    for (int st = 0; st < nst; ++st) {
      __syncthreads();   // the previous stage's LDS readers are done
#pragma unroll
      for (int j = 0; j < kWJ; ++j) {
        uint32_t* dst = T + ((lr + 8 * j) * kPitch + 8 * lc) / 2;
        dst[0] = v[j].x; dst[1] = v[j].y; dst[2] = v[j].z; dst[3] = v[j].w;
      }
      {
        float av[kAR];
#pragma unroll
        for (int e = 0; e < kAR; ++e) {
          const bool keep = tok_ok && st * kKT + kAR * ar + e < nseg && (!has_mask || mb[e] != 0u);
          av[e] = keep ? xr[e] : 0.f;
        }
        uint32_t hi[kAR / 2], lo[kAR / 2];
#pragma unroll
        for (int e = 0; e < kAR / 2; ++e) {
          const uint32_t h0 = f32_to_bf16_rne(av[2 * e]), h1 = f32_to_bf16_rne(av[2 * e + 1]);
          const uint32_t l0 = f32_to_bf16_rne(av[2 * e] - __uint_as_float(h0 << 16));
          const uint32_t l1 = f32_to_bf16_rne(av[2 * e + 1] - __uint_as_float(h1 << 16));
          hi[e] = h0 | (h1 << 16);
          lo[e] = l0 | (l1 << 16);
        }
        uint32_t* ah = reinterpret_cast<uint32_t*>(&As[0][am][0]) + (kAR / 2) * ar;
        uint32_t* al = reinterpret_cast<uint32_t*>(&As[1][am][0]) + (kAR / 2) * ar;
#pragma unroll
        for (int e = 0; e < kAR / 2; ++e) { ah[e] = hi[e]; al[e] = lo[e]; }
      }
      if (st + 1 < nst) issue(st + 1);   // in flight while this stage is contracted
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kKT / 32; ++s) {
        const bf16x8 Ah = __builtin_bit_cast(bf16x8, As[0][nl][4 * s + g]);
        const bf16x8 Al = __builtin_bit_cast(bf16x8, As[1][nl][4 * s + g]);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int o = 64 * w + 16 * nt + nl;
          const uint16_t* src = Ts + (32 * s + 8 * g) * kPitch + o;
          uint32_t b[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            b[jj] = (uint32_t)src[(2 * jj) * kPitch] | ((uint32_t)src[(2 * jj + 1) * kPitch] << 16);
          const bf16x8 Bv = __builtin_bit_cast(bf16x8, make_uint4(b[0], b[1], b[2], b[3]));
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ah, Bv, acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Al, Bv, acc[nt], 0, 0, 0);
        }
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
  const int col_tiles = (a.d + kOT - 1) / kOT;
  // one round of workgroups, two per CU on 256 CUs (measured on the 17408 x
  // 5120 union at batch 16 with 64-row stages: 512 workgroups 46.0 us, 768
  // 49.4, 384 53.6; with 32-row stages 512: 41.9, 256: 52.3, 1024: 45.3;
  // fewer chunks also shrink the partials' round trip)
  long KS = 512 / ((long)col_tiles * Mt);
  const long by_rows = (items + kKT - 1) / kKT;
  if (KS > by_rows) KS = by_rows;
  if (KS > max_split_mfma(Mt)) KS = max_split_mfma(Mt);
  if (KS < 1) KS = 1;
  float* partials = reinterpret_cast<float*>(reinterpret_cast<char*>(a.ws) + kWsHeaderBytes);
  hipLaunchKernelGGL(axpy_mfma_kernel, dim3(col_tiles, (int)KS, Mt), dim3(256), 0, s, a, (int)KS,
                     Mpad, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_splitk_reduce(partials, (int)KS, a.batch, Mpad, a.d, a.alpha, a.out, a.ld_out,
                              a.accumulate, s);
}

}  // namespace sffn
