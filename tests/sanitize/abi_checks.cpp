// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the library's argument-validation layer
// (tests/test_abi_sanitized.py builds and runs it; no GPU is used: every
// call below is rejected before anything is launched, or is a pure size
// query).  Each case checks the returned status and that sffn_last_error()
// names the problem; a second part provokes different errors on several
// host threads at once and checks that each thread reads back its own
// message (the error text is thread-local).
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "sparse_ffn.h"

namespace {

int failures = 0;
void* const FAKE = reinterpret_cast<void*>(0x1000);   // never dereferenced
void* const MIS4 = reinterpret_cast<void*>(0x1004);   // 4-byte but not 16-byte aligned

void expect(const char* what, int rc, int want, const char* needle) {
  const std::string msg = sffn_last_error();
  const bool ok = rc == want && (needle == nullptr || msg.find(needle) != std::string::npos);
  if (!ok) {
    std::printf("FAIL %s: status %d (want %d), message \"%s\" (want \"%s\")\n", what, rc, want,
                msg.c_str(), needle ? needle : "");
    ++failures;
  }
}

const uint16_t* W(void* p = FAKE) { return static_cast<const uint16_t*>(p); }
const float* F(void* p = FAKE) { return static_cast<const float*>(p); }
float* Fo(void* p = FAKE) { return static_cast<float*>(p); }
const int32_t* I(void* p = FAKE) { return static_cast<const int32_t*>(p); }

int gemv(int op, int n_rows, int d, int ld_w, int batch, const int32_t* idx, const int32_t* count,
         int k_max, int group, void* ws, size_t ws_bytes, const float* in = F(),
         const uint16_t* W1 = W(), float tau = 0.f, float eps = 0.f, const float* aux = nullptr,
         int ld_aux = 0, int ld_out = 64, int ld_in = 64) {
  return sparse_ffn_gemv(op, W(), W1, n_rows, d, ld_w, in, batch, ld_in, idx, count, k_max, group,
                         nullptr, 0, tau, eps, aux, ld_aux, nullptr, Fo(), nullptr, ld_out, 0, ws,
                         ws_bytes, nullptr);
}

int select(const void* keys, int key_type, int n, int ld, int cluster, int r_lo, int r_hi,
           int nz = 0, int32_t* idx = nullptr, int ld_idx = 0, const float* scale = nullptr,
           int clear = 0, uint32_t* freq = nullptr) {
  return sparse_ffn_select(keys, key_type, scale, 1, n, ld, cluster, r_lo, r_hi, nz, nullptr,
                           nullptr, nullptr, 0, idx, ld_idx, nullptr, nullptr, 0, nullptr, freq,
                           clear, nullptr);
}

void single_thread_cases() {
  // sizes
  if (sffn_abi_version() != SFFN_ABI_VERSION) { std::printf("FAIL abi version\n"); ++failures; }
  if (sparse_ffn_tier_record_bytes(6144, 3) != 16 + 3072) { std::printf("FAIL record bytes\n"); ++failures; }
  if (sparse_ffn_tier_record_bytes(4096, 5) != 0) { std::printf("FAIL record bytes n_seg\n"); ++failures; }
  if (sparse_ffn_workspace_size(1, 4096, 2048) < (size_t)256 * 2048 * 4) { std::printf("FAIL ws size\n"); ++failures; }
  if (sparse_ffn_workspace_size(-3, -1, -1) == 0) { std::printf("FAIL ws size of bad shape\n"); ++failures; }

  // select
  expect("select null keys", select(nullptr, 0, 8, 8, 1, 0, 4), SFFN_EINVAL, "keys");
  expect("select n", select(FAKE, 0, 40000, 40000, 1, 0, 4), SFFN_EUNSUPPORTED, "32768");
  expect("select ld", select(FAKE, 0, 8, 4, 1, 0, 4), SFFN_EINVAL, "ld");
  expect("select r_lo", select(FAKE, 0, 8, 8, 1, 5, 4), SFFN_EINVAL, "r_lo");
  expect("select signed nz", select(FAKE, 2, 8, 8, 1, 0, 4, 1), SFFN_EINVAL, "signed");
  expect("select key type", select(FAKE, 7, 8, 8, 1, 0, 4), SFFN_EINVAL, "key type");
  expect("select cluster 0", select(FAKE, 0, 8, 8, 0, 0, 4), SFFN_EINVAL, "cluster");
  expect("select n*cluster", select(FAKE, 0, 8, 16, 4, 0, 4), SFFN_EINVAL, "n*cluster");
  expect("select clusters", select(FAKE, 0, 5000, 10000, 2, 0, 4), SFFN_EUNSUPPORTED, "4096");
  expect("select 2^30", select(FAKE, 0, 4096, 2147483647, (1 << 18) + 1, 0, 4), SFFN_EUNSUPPORTED,
         "2^30");
  expect("select ld_idx", select(FAKE, 0, 8, 8, 1, 0, 4, 0, static_cast<int32_t*>(FAKE), 3),
         SFFN_EINVAL, "ld_idx");
  expect("select scale type", select(FAKE, 1, 8, 8, 1, 0, 4, 0, nullptr, 0, F()), SFFN_EINVAL,
         "key_scale");
  expect("select clear+freq", select(FAKE, 1, 8, 8, 1, 0, 4, 0, nullptr, 0, nullptr, 1,
                                     static_cast<uint32_t*>(FAKE)), SFFN_EINVAL, "clear_keys");

  // gemv
  expect("gemv op", gemv(9, 64, 64, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0), SFFN_EINVAL, "op");
  expect("gemv d", gemv(3, 64, 12, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0), SFFN_EINVAL,
         "multiple of 8");
  expect("gemv ld_w", gemv(3, 64, 64, 60, 1, nullptr, nullptr, 0, 1, nullptr, 0), SFFN_EINVAL, "ld_w");
  expect("gemv batch d%32", gemv(3, 64, 40, 40, 2, nullptr, nullptr, 0, 1, nullptr, 0, F(), W(),
                                 0.f, 0.f, nullptr, 0, 40, 64), SFFN_EUNSUPPORTED, "d % 32");
  expect("gemv align", gemv(3, 64, 64, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0, F(MIS4)),
         SFFN_EINVAL, "aligned");
  expect("gemv count", gemv(3, 64, 64, 64, 1, I(), nullptr, 4, 1, nullptr, 0), SFFN_EINVAL, "count");
  expect("gemv k_max", gemv(3, 64, 64, 64, 1, I(), I(), 3, 32, nullptr, 0), SFFN_EINVAL, "exceeds");
  expect("gemv workspace", gemv(3, 64, 64, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0),
         SFFN_EWORKSPACE, "workspace");
  expect("gemv small ws", gemv(3, 64, 64, 64, 1, nullptr, nullptr, 0, 1, FAKE, 100),
         SFFN_EWORKSPACE, nullptr);
  expect("gemv W1", gemv(0, 64, 64, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0, F(), nullptr),
         SFFN_EINVAL, "W1");
  expect("gemv tau", gemv(1, 64, 64, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0, F(), W(), -1.f),
         SFFN_EINVAL, "tau");
  expect("gemv wide row", gemv(0, 64, 8200, 8200, 1, nullptr, nullptr, 0, 1, nullptr, 0, F(), W(),
                               0.f, 0.f, nullptr, 0, 64, 8200), SFFN_EUNSUPPORTED, "8192");
  expect("gemv predict theta", gemv(6, 64, 64, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0, F(), W(),
                                    1.5f), SFFN_EINVAL, "probability");
  expect("gemv relu cluster idx", gemv(7, 64, 64, 64, 1, I(), I(), 2, 32, nullptr, 0),
         SFFN_EUNSUPPORTED, "idx must be NULL");

  // the allocation-free gemv: scratch limit checked before any device call
  expect("noalloc limit",
         sparse_ffn_gemv_noalloc(3, W(), nullptr, 64, 1 << 16, 1 << 16, F(), 1, 64, nullptr,
                                 nullptr, 0, 1, nullptr, 0, 0.f, 0.f, nullptr, 0, nullptr, Fo(),
                                 nullptr, 1 << 16, 0, nullptr),
         SFFN_EWORKSPACE, "static");
  expect("noalloc row op",
         sparse_ffn_gemv_noalloc(0, W(), nullptr, 64, 64, 64, F(), 1, 64, nullptr, nullptr, 0, 1,
                                 nullptr, 0, 0.f, 0.f, nullptr, 0, nullptr, Fo(), nullptr, 64, 0,
                                 nullptr),
         SFFN_EINVAL, "W1");

  // lists
  const uint16_t* Ws[2] = {W(), W()};
  const float* ins[2] = {F(), F()};
  const int32_t* idxs[2] = {I(), I()};
  const int32_t* cnts[2] = {I(), I()};
  int nr[2] = {64, 64}, km[2] = {2, 3};
  expect("lists n", sparse_ffn_gemv_lists(9, Ws, nr, 64, 64, ins, idxs, cnts, km, 32, nullptr,
                                          Fo(), 1, FAKE, 1 << 30, nullptr), SFFN_EINVAL, "n_lists");
  expect("lists k_max", sparse_ffn_gemv_lists(2, Ws, nr, 64, 64, ins, idxs, cnts, km, 32, nullptr,
                                              Fo(), 1, FAKE, 1 << 30, nullptr), SFFN_EINVAL,
         "exceeds");
  expect("lists host arrays", sparse_ffn_gemv_lists(2, nullptr, nr, 64, 64, ins, idxs, cnts, km,
                                                    32, nullptr, Fo(), 1, FAKE, 1 << 30, nullptr),
         SFFN_EINVAL, "host arrays");
  float* outs[2] = {Fo(), Fo()};
  expect("rowop lists op", sparse_ffn_rowop_lists(3, 2, Ws, Ws, 64, 64, 64, F(), nullptr, nullptr,
                                                  nullptr, 1, 0.f, 0.f, nullptr, outs, nullptr, 0,
                                                  nullptr), SFFN_EINVAL, "not a row op");
  expect("rowop lists d", sparse_ffn_rowop_lists(0, 2, Ws, Ws, 64, 5128, 5128, F(), nullptr,
                                                 nullptr, nullptr, 1, 0.f, 0.f, nullptr, outs,
                                                 nullptr, 0, nullptr), SFFN_EUNSUPPORTED, "5120");

  // score, tiers, compaction, gather, norms
  expect("score mode", sparse_ffn_score(5, F(), 1, 8, 8, 1, 0, nullptr, 0, FAKE, nullptr),
         SFFN_EINVAL, nullptr);
  expect("score cluster", sparse_ffn_score(1, F(), 1, 100, 100, 32, 0, nullptr, 0, FAKE, nullptr),
         SFFN_EINVAL, "multiple");
  const int32_t seg[4] = {0, 4096, 5120, 6144}, bad[4] = {0, 4000, 5120, 6144};
  expect("encode seg", sparse_ffn_encode_tiers(W(), 6144, 16, 6144, bad, 3,
                                               static_cast<uint8_t*>(FAKE), 3088, nullptr),
         SFFN_EINVAL, "multiple of 64");
  expect("encode rec", sparse_ffn_encode_tiers(W(), 6144, 16, 6144, seg, 3,
                                               static_cast<uint8_t*>(FAKE), 3072, nullptr),
         SFFN_EINVAL, "rec_bytes");
  expect("tiered ws", sparse_ffn_tiered_gemv(W(), 6144, static_cast<const uint8_t*>(FAKE), 3088,
                                             seg, 3, 4096, 6144, F(), I(), I(), 614, I(), I(),
                                             1433, Fo(), 0, FAKE, 64, nullptr),
         SFFN_EWORKSPACE, "workspace");
  expect("compact k", sparse_ffn_compact(W(), 100, 64, 64, I(), 101, 0,
                                         static_cast<uint16_t*>(FAKE), 64, nullptr),
         SFFN_EINVAL, "k=");
  expect("norms d", sparse_ffn_row_norms(W(), 8, 60, 64, Fo(), nullptr), SFFN_EINVAL,
         "multiple of 8");

  // fused per-neuron SwiGLU
  auto fused = [](const uint16_t* Wd, int d, int ld_w, float eps, const int32_t* idx,
                  const int32_t* cnt, int k_max, void* ws, size_t ws_bytes) {
    return sparse_ffn_fused_swiglu(W(), W(), Wd, 64, d, ld_w, F(), eps, idx, cnt, k_max, nullptr,
                                   Fo(), 1, ws, ws_bytes, nullptr);
  };
  expect("fused Wd", fused(nullptr, 64, 192, 0.f, nullptr, nullptr, 0, FAKE, 1 << 30), SFFN_EINVAL,
         "Wd");
  expect("fused align", fused(W(MIS4), 64, 192, 0.f, nullptr, nullptr, 0, FAKE, 1 << 30),
         SFFN_EINVAL, "16-byte");
  expect("fused d", fused(W(), 4104, 12312, 0.f, nullptr, nullptr, 0, FAKE, 1 << 30),
         SFFN_EUNSUPPORTED, "4096");
  expect("fused eps", fused(W(), 64, 192, -1.f, nullptr, nullptr, 0, FAKE, 1 << 30), SFFN_EINVAL,
         "rms_eps");
  expect("fused count", fused(W(), 64, 192, 0.f, I(), nullptr, 4, FAKE, 1 << 30), SFFN_EINVAL,
         "count");
  expect("fused k_max", fused(W(), 64, 192, 0.f, I(), I(), 65, FAKE, 1 << 30), SFFN_EINVAL,
         "k_max");
  expect("fused workspace", fused(W(), 64, 192, 0.f, nullptr, nullptr, 0, nullptr, 0),
         SFFN_EWORKSPACE, "workspace");

  // packed layouts and the gemv flag
  if (sparse_ffn_packed_elems(1000, 384, SFFN_LAYOUT_ROW_TILES) != (size_t)1008 * 384) {
    std::printf("FAIL packed elems\n"); ++failures;
  }
  uint16_t* const OUT = static_cast<uint16_t*>(reinterpret_cast<void*>(0x100000));
  expect("pack layout", sparse_ffn_pack_weights(W(), 64, 384, 384, 3, OUT, nullptr), SFFN_EINVAL,
         "layout");
  expect("pack d", sparse_ffn_pack_weights(W(), 64, 384, 384, SFFN_LAYOUT_COL_PANELS, OUT, nullptr),
         SFFN_EINVAL, "multiple of 256");
  expect("pack overlap", sparse_ffn_pack_weights(W(), 64, 256, 256, SFFN_LAYOUT_ROW_TILES,
                                                 static_cast<uint16_t*>(FAKE), nullptr),
         SFFN_EINVAL, "overlaps");
  expect("packed batch 1", gemv(SFFN_OP_GLU_SILU | SFFN_PACKED, 64, 128, 128, 1, nullptr, nullptr,
                                0, 1, nullptr, 0, F(), W(), 0.f, 0.f, nullptr, 0, 64, 128),
         SFFN_EUNSUPPORTED, "batch > 1");
  expect("packed axpy d", gemv(SFFN_OP_AXPY | SFFN_PACKED, 64, 384, 384, 4, nullptr, nullptr, 0, 1,
                               FAKE, 1 << 30, F(), W(), 0.f, 0.f, nullptr, 0, 384, 64),
         SFFN_EUNSUPPORTED, "256");

  // the union formed in the product (masked rows)
  auto masked = [](int batch, const int32_t* idx, const uint8_t* mask, int ld_mask) {
    return sparse_ffn_gemv(SFFN_OP_AXPY | SFFN_MASKED_ROWS, W(), nullptr, 64, 256, 256, F(), batch,
                           64, idx, idx ? I() : nullptr, idx ? 4 : 0, 1, mask, ld_mask, 0.f, 0.f,
                           nullptr, 0, nullptr, Fo(), nullptr, 256, 0, FAKE, 1 << 30, nullptr);
  };
  const uint8_t* MK = static_cast<const uint8_t*>(FAKE);
  expect("masked batch", masked(1, nullptr, MK, 64), SFFN_EUNSUPPORTED, "batch > 1");
  expect("masked mask", masked(4, nullptr, nullptr, 0), SFFN_EINVAL, "row_mask");
  expect("masked idx", masked(4, I(), MK, 64), SFFN_EINVAL, "idx must be NULL");
  expect("masked ld", masked(4, nullptr, MK, 72), SFFN_EINVAL, "ld_mask");

  // the top-k range as a threshold pair, and the product keyed by it
  uint32_t* const THR = static_cast<uint32_t*>(reinterpret_cast<void*>(0x1008));
  expect("thr keys", sparse_ffn_select_threshold(nullptr, 1, 1, 8, 8, 0, 4, nullptr, THR, nullptr), SFFN_EINVAL,
         "keys");
  expect("thr n", sparse_ffn_select_threshold(FAKE, 1, 1, 40000, 40000, 0, 4, nullptr, THR, nullptr),
         SFFN_EUNSUPPORTED, "32768");
  expect("thr k", sparse_ffn_select_threshold(FAKE, 1, 1, 8, 8, 0, -1, nullptr, THR, nullptr), SFFN_EINVAL,
         "k=");
  expect("thr align", sparse_ffn_select_threshold(FAKE, 1, 1, 8, 8, 0, 4, nullptr,
                                                  static_cast<uint32_t*>(MIS4), nullptr),
         SFFN_EINVAL, "8-byte");
  expect("thr k_top", sparse_ffn_select_threshold(FAKE, 1, 1, 8, 8, 5, 4, THR, THR, nullptr),
         SFFN_EINVAL, "k_top=5");
  expect("thr top", sparse_ffn_select_threshold(FAKE, 1, 1, 8, 8, 2, 4, nullptr, THR, nullptr),
         SFFN_EINVAL, "needs thr_top_out");
  auto keyed = [](const uint16_t* Wk, int n_rows, int d, int k_max, const uint32_t* thr, void* ws,
                  size_t ws_bytes) {
    return sparse_ffn_gemv_keyed(Wk, n_rows, d, d, F(), FAKE, 1, thr, k_max, nullptr, Fo(), 0, ws,
                                 ws_bytes, nullptr);
  };
  void* const WS = reinterpret_cast<void*>(0x100000);
  expect("keyed W", keyed(nullptr, 64, 256, 32, THR, WS, 1 << 30), SFFN_EINVAL, "W must");
  expect("keyed thr", keyed(W(), 64, 256, 32, static_cast<uint32_t*>(MIS4), WS, 1 << 30),
         SFFN_EINVAL, "thr");
  expect("keyed k_max", keyed(W(), 64, 256, 65, THR, WS, 1 << 30), SFFN_EINVAL, "k_max");
  expect("keyed rows", keyed(W(), 270000, 256, 10, THR, WS, 1 << 30), SFFN_EUNSUPPORTED, "chunks");
  expect("keyed workspace", keyed(W(), 64, 256, 32, THR, nullptr, 0), SFFN_EWORKSPACE, "workspace");
  const int32_t seg_k[4] = {0, 4096, 5120, 6144};
  auto tk = [&](int n_in, const uint32_t* thr_top, size_t ws_bytes) {
    return sparse_ffn_tiered_gemv_keyed(W(), 6144, static_cast<const uint8_t*>(FAKE), 3088, seg_k,
                                        3, n_in, 6144, F(), FAKE, 0, thr_top, THR, 10, 10, Fo(), 0, WS,
                                        ws_bytes, nullptr);
  };
  expect("tiered keyed n_in", tk(600000, THR, 1 << 30), SFFN_EUNSUPPORTED, "524288");
  expect("tiered keyed thr", tk(4096, nullptr, 1 << 30), SFFN_EINVAL, "thr_top");
  expect("tiered keyed workspace", tk(4096, THR, 64), SFFN_EWORKSPACE, "workspace");
}

// Several threads provoke different errors at once; each must read back the
// message of its own last call.
void thread_cases() {
  std::vector<std::thread> th;
  std::vector<int> bad(8, 0);
  for (int t = 0; t < 8; ++t) {
    th.emplace_back([t, &bad] {
      for (int it = 0; it < 2000; ++it) {
        int rc;
        const char* needle;
        if (t % 2 == 0) {
          rc = select(nullptr, 0, 8, 8, 1, 0, 4);
          needle = "keys";
        } else {
          rc = gemv(3, 64, 12, 64, 1, nullptr, nullptr, 0, 1, nullptr, 0);
          needle = "multiple of 8";
        }
        if (rc != SFFN_EINVAL || std::strstr(sffn_last_error(), needle) == nullptr) ++bad[t];
      }
    });
  }
  for (auto& x : th) x.join();
  for (int t = 0; t < 8; ++t)
    if (bad[t]) { std::printf("FAIL thread %d read another thread's error %d times\n", t, bad[t]); ++failures; }
}

}  // namespace

int main() {
  single_thread_cases();
  thread_cases();
  std::printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
