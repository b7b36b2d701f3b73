// Device helpers and launcher declarations shared by the HIP kernels of
// libsparse_ffn.so.  Internal to the library; the public surface is
// include/sparse_ffn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sffn {

constexpr int kWave = 64;

// ----------------------------------------------------------------- bf16 / keys

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Eight bf16 values packed in a uint4 -> fp32, in memory order.
__device__ __forceinline__ void unpack8(const uint4& w, float (&f)[8]) {
  f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
  f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
  f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
  f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// Magnitude key: fp32 bits with the sign cleared (orders |v|).
__device__ __forceinline__ uint32_t key_abs(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Order-preserving key of a signed fp32 value.
__device__ __forceinline__ uint32_t key_signed(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Round fp32 to bf16 (nearest-even) and return the bits; finite inputs.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Wave index within the workgroup as a wave-uniform (scalar) value, so loops
// bounded by it stay scalar loops rather than exec-masked ones.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// ----------------------------------------------------------------- wave reductions

// Sum over the 64 lanes with DPP lane moves (no LDS round trips): pairs and
// quads, then the 8- and 16-lane mirrors, then the row broadcasts of lanes
// 15 and 31 fold the four 16-lane rows into lane 63, which is read back as a
// wave-uniform value.  Call with every lane of the wave active.
#define SFFN_DPP_ADD(v, ctrl)                                                              \
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xf, 0xf, false))
#define SFFN_DPP_ADD_ROWS(v, ctrl, rows)                                                   \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rows, 0xf, false))
__device__ __forceinline__ float wave_sum(float v) {
  SFFN_DPP_ADD(v, 0xB1);              // quad_perm [1,0,3,2]
  SFFN_DPP_ADD(v, 0x4E);              // quad_perm [2,3,0,1]
  SFFN_DPP_ADD(v, 0x141);             // row_half_mirror
  SFFN_DPP_ADD(v, 0x140);             // row_mirror: every lane holds its 16-lane row sum
  SFFN_DPP_ADD_ROWS(v, 0x142, 0xa);   // row_bcast:15 into rows 1 and 3
  SFFN_DPP_ADD_ROWS(v, 0x143, 0xc);   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
#undef SFFN_DPP_ADD
#undef SFFN_DPP_ADD_ROWS

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// ----------------------------------------------------------------- workspace layout
// [header: kWsHeaderBytes][partials: fp32][packed activations: bf16 hi/lo]
constexpr size_t kWsHeaderBytes = 256;
constexpr int kMaxSplit = 256;               // largest split-K factor

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ----------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already validated.

struct RowOpArgs {
  int op;
  const uint16_t* W0; const uint16_t* W1;
  int n_rows, d, ld_w;
  const float* x; int batch, ld_in;
  const int32_t* idx; const int32_t* count; int k_max, group;
  float tau_scale, rms_eps;
  const float* aux; int ld_aux;
  float* out; uint32_t* key_out; int ld_out; int accumulate;
  void* ws; size_t ws_bytes;   // optional (batched row ops: K split of the last tiles)
  int packed;                  // W0 / W1 in the row-tile layout (batched kernel only)
};
hipError_t launch_rowop_b1(const RowOpArgs& a, hipStream_t s);
hipError_t launch_rowop_mfma(const RowOpArgs& a, hipStream_t s);

// A row op over several row lists at batch 1 (e.g. the routed experts of a
// MoE layer): list l reads W0[l] / W1[l] at its rows and writes out[l],
// key_out[l]; the shared fields (op, shape, x, group, tau_scale, rms_eps)
// come from `base`, whose per-list fields are unused.
constexpr int kMaxRowLists = 8;
struct RowOpListsArgs {
  RowOpArgs base;
  int n;
  const uint16_t* W0[kMaxRowLists];
  const uint16_t* W1[kMaxRowLists];
  const int32_t* idx[kMaxRowLists];
  const int32_t* count[kMaxRowLists];
  int k_max[kMaxRowLists];
  const float* aux[kMaxRowLists];
  float* out[kMaxRowLists];
  uint32_t* key_out[kMaxRowLists];
};
hipError_t launch_rowop_lists(const RowOpListsArgs& a, hipStream_t s);

struct AxpyArgs {
  const uint16_t* W; int n_rows, d, ld_w;
  const float* in; int batch, ld_in;
  const int32_t* idx; const int32_t* count; int k_max, group;
  const uint8_t* row_mask; int ld_mask;
  const float* alpha;
  float* out; int ld_out; int accumulate;
  void* ws; size_t ws_bytes;
  int packed;                  // W in the column-panel layout (batched kernel only)
  int mask_rows;               // no index list: the rows some token's mask selects (batched)
};
hipError_t launch_axpy_b1(const AxpyArgs& a, hipStream_t s);
hipError_t launch_axpy_mfma(const AxpyArgs& a, hipStream_t s);
// The batch-1 gathered product over the rows a threshold (T, I) selects:
// row n is read iff key_n > T, or key_n == T and n <= I (key_n = keys[n]
// read as key_type); AxpyArgs.idx / count are unused, k_max bounds the
// selected count (launch shape only).
hipError_t launch_axpy_keyed(const AxpyArgs& a, const void* keys, int key_type,
                             const uint32_t* thr, hipStream_t s);

// Gathered products over several row lists into one output at batch 1.
constexpr int kMaxLists = 8;
struct AxpyList {
  const uint16_t* W; const float* in; const int32_t* idx; const int32_t* count;
  const float* alpha; int k_max;
};
struct AxpyListsArgs {
  AxpyList l[kMaxLists];
  int n, d, ld_w, group;
  float* out; int accumulate;
  void* ws; size_t ws_bytes;
};
hipError_t launch_axpy_lists(const AxpyListsArgs& a, hipStream_t s);

struct SelectArgs {
  const void* keys; int key_type; const float* key_scale; int rows, n, ld, cluster;
  int r_lo, r_hi, nonzero_only;
  const uint8_t* include_mask;
  const uint8_t* exclude_mask;
  uint8_t* mask_out; int ld_mask;
  int32_t* idx_out; int ld_idx;
  int32_t* count_out;
  int32_t* idx_top_out; int ld_idx_top;
  int32_t* count_top_out;
  uint32_t* freq;
  int clear_keys;
  uint32_t* thr_out;       // threshold mode (no lists): (T, I) of the range [0, r_hi) per row
  uint32_t* thr_top_out;   // and, if set, (T, I) of [0, r_lo)
};
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

hipError_t launch_score(int mode, const float* in, int T, int n, int ld, int cluster,
                        int accumulate, const int32_t* picked, int k, void* out,
                        hipStream_t s);
hipError_t launch_row_norms(const uint16_t* W, int n_rows, int d, int ld_w, float* out,
                            hipStream_t s);

struct TierArgs {
  const uint16_t* Wt; int ld_w;
  const uint8_t* rec; int rec_bytes;
  int seg_bounds[5]; int n_seg;
  int n_in, d_out;
  const float* x;
  const int32_t* idx_top; const int32_t* cnt_top; int k_top_max;
  const int32_t* idx_mid; const int32_t* cnt_mid; int k_mid_max;
  float* y; int accumulate;
  void* ws; size_t ws_bytes;
  // keyed tiers (thr set, idx_* unused): the top tier is the set of thr_top,
  // the middle tier the set of thr less the top tier; keys read as key_type
  const void* keys; int key_type;
  const uint32_t* thr_top; const uint32_t* thr;
};
hipError_t launch_tiered(const TierArgs& a, hipStream_t s);
int tiered_keyed_min_chunks(int n_in);
hipError_t launch_encode_tiers(const uint16_t* Wt, int ld_w, int n_in, int d_out,
                               const int* seg_bounds, int n_seg, uint8_t* rec,
                               int rec_bytes, hipStream_t s);

// Fused sparse-SwiGLU decode at batch 1: gate, up, silu * mul and the down
// row of every processed neuron in one pass; workgroup partials of y in the
// workspace, added in order by the split-K reduction.
struct FusedArgs {
  const uint16_t* Wg; const uint16_t* Wu; const uint16_t* Wd; int ld_w;
  int n_rows, d;
  const float* x; float rms_eps;
  const int32_t* idx; const int32_t* count; int k_max;
  float* a_out; float* y; int accumulate;
  void* ws; size_t ws_bytes;
};
hipError_t launch_fused_swiglu(const FusedArgs& a, hipStream_t s);

// Packed weight layouts of the batched (MFMA) kernels.
//  row tiles   : element (r, k) at ((r / 16) * (d / 128) + k / 128) * 2048
//                + (r % 16) * 128 + k % 128; rows padded to a multiple of 16
//                with zeros (d % 128 == 0).
//  col panels  : element (r, o) at (o / 256) * n * 256 + r * 256 + o % 256
//                (d % 256 == 0).
constexpr int kLayoutRowTiles = 1;
constexpr int kLayoutColPanels = 2;
size_t packed_elems(int n_rows, int d, int layout);
hipError_t launch_pack(const uint16_t* W, int n_rows, int d, int ld_w, int layout, uint16_t* out,
                       hipStream_t s);

hipError_t launch_compact(const uint16_t* W, int ld_w, int d, const int32_t* idx, int k,
                          int transpose, uint16_t* out, int ld_out, hipStream_t s);
hipError_t launch_gather32(const uint32_t* src, int n_src, const int32_t* idx,
                           const int32_t* count, int k_max, uint32_t* dst, hipStream_t s);

size_t workspace_bytes(int batch, int n_rows, int d_out);
int pick_split_b1(long items, int col_tiles);
int keyed_split(int n_rows, long k_max, int col_tiles);
int max_split_mfma(int mtiles);

}  // namespace sffn
