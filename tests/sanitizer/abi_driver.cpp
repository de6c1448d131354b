// Drives every entry point of include/fa.h through its argument checks and,
// with valid arguments, through to the (stubbed) launcher, under ASan/UBSan.
// Fake device pointers are never dereferenced: validation only compares them
// and the stubs only record them. Exits non-zero on the first mismatch.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "fa.h"
#include "fa_launch.h"

namespace fa {
extern FwdParams g_fwd;
extern BwdParams g_bwd;
extern DecodeParams g_dec;
extern Fp8QuantParams g_q8;
extern Fp8FwdParams g_f8;
extern int g_calls;
}

static int g_fail = 0;
#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                    \
      std::fprintf(stderr, "\n");                           \
      ++g_fail;                                             \
    }                                                       \
  } while (0)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static const uintptr_t B = 0x100000000ull;   // fake device addresses, 16-byte aligned, far apart

static void check(fa_status_t got, fa_status_t want, const char* what) {
  EXPECT(got == want, "%s: status %d, expected %d (%s)", what, (int)got, (int)want, fa_last_error_message());
  if (want != FA_OK) EXPECT(std::strlen(fa_last_error_message()) > 0, "%s: empty error message", what);
  else EXPECT(fa_last_error_message()[0] == 0, "%s: message left after success", what);
}

static void fwd_cases() {
  const int64_t qs[3] = {64 * 256 * 128, 256 * 128, 128}, ks[3] = {8 * 256 * 128, 256 * 128, 128};
  auto call = [&](const void* q, int hq, int hkv, int nq, int nk, int d, const int64_t* s, int in, int out, int mask,
                  float scale) {
    return fa_fwd(q, P(B * 2), P(B * 3), P(B * 4), (float*)P(B * 5), 1, hq, hkv, nq, nk, d, s, ks, ks, s,
                  (fa_dtype_t)in, (fa_dtype_t)out, (fa_mask_t)mask, scale, nullptr);
  };
  check(call(P(B), 64, 8, 256, 256, 128, qs, 0, 0, 1, 0.088f), FA_OK, "fwd valid");
  EXPECT(fa::g_fwd.heads_q == 64 && fa::g_fwd.group == 8 && fa::g_fwd.causal && fa::g_fwd.q_stride[1] == qs[1],
         "fwd params");
  check(call(nullptr, 64, 8, 256, 256, 128, qs, 0, 0, 1, 0.088f), FA_ERR_INVALID_ARGUMENT, "fwd null q");
  check(call(P(B), 64, 8, 256, 256, 96, qs, 0, 0, 1, 0.088f), FA_ERR_UNSUPPORTED, "fwd d=96");
  check(call(P(B), 64, 7, 256, 256, 128, qs, 0, 0, 0, 0.088f), FA_ERR_UNSUPPORTED, "fwd Hq%Hkv");
  check(call(P(B), 64, 8, 256, 300, 128, qs, 0, 0, 1, 0.088f), FA_ERR_UNSUPPORTED, "fwd causal Nq!=Nk");
  check(call(P(B + 8), 64, 8, 256, 256, 128, qs, 0, 0, 1, 0.088f), FA_ERR_UNSUPPORTED, "fwd misaligned");
  check(call(P(B), 64, 8, 256, 256, 128, qs, 0, 0, 1, NAN), FA_ERR_INVALID_ARGUMENT, "fwd nan scale");
  check(call(P(B), 64, 8, 256, 256, 128, qs, 9, 0, 1, 0.1f), FA_ERR_INVALID_ARGUMENT, "fwd dtype");
  check(call(P(B), 64, 8, 256, 256, 128, nullptr, 0, 0, 1, 0.1f), FA_ERR_INVALID_ARGUMENT, "fwd strides");
  {  // sizes whose products overflow 32 bits: refused, with no signed overflow on the way (UBSan)
    const fa_status_t st = fa_fwd(P(B), P(B * 2), P(B * 3), P(B * 4), nullptr, 0x7fff, 64, 8, 0x7fffffff, 0x7fffffff,
                                  128, qs, ks, ks, qs, FA_DTYPE_BF16, FA_DTYPE_BF16, FA_MASK_NONE, 0.1f, nullptr);
    EXPECT(st != FA_OK, "fwd huge sizes accepted");
  }
  // varlen
  const int64_t vs[2] = {64 * 128, 128}, kvs[2] = {8 * 128, 128};
  check(fa_fwd_varlen(P(B), P(B * 2), P(B * 3), P(B * 4), nullptr, (const int32_t*)P(B * 6), 3, 64, 8, 1000, 600,
                      128, vs, kvs, kvs, vs, FA_DTYPE_BF16, FA_MASK_CAUSAL, 100, 0.088f, nullptr),
        FA_OK, "varlen valid");
  EXPECT(fa::g_fwd.window == 100 && fa::g_fwd.total == 1000 && fa::g_fwd.cu_seqlens != nullptr, "varlen params");
  check(fa_fwd_varlen(P(B), P(B * 2), P(B * 3), P(B * 4), nullptr, (const int32_t*)P(B * 6), 3, 64, 8, 1000, 600,
                      128, vs, kvs, kvs, vs, FA_DTYPE_BF16, FA_MASK_NONE, 100, 0.088f, nullptr),
        FA_ERR_UNSUPPORTED, "varlen window without causal");
}

static void decode_cases() {
  const int64_t kv[3] = {8 * 4096 * 128, 4096 * 128, 128};
  for (int d : {64, 128}) {
    const int64_t kvd[3] = {8 * 4096 * d, 4096 * d, d};
    const size_t ws = fa_decode_workspace_bytes(16, 64, 8, 4096, d, 0);
    EXPECT(ws > 0 && ws == fa_decode_workspace_bytes(16, 64, 8, 4096, d, 999), "workspace independent of split");
    std::vector<char> dummy;   // bounds of the partials are checked against [B*7, B*7 + ws)
    check(fa_decode(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 4), P(B * 5), nullptr, 16, 64, 8, 4096, d, kvd,
                    FA_DTYPE_FP32, 0.088f, 0, P(B * 7), ws, nullptr),
          FA_OK, "decode valid");
    const char* lo = (const char*)P(B * 7);
    const int64_t parts = ((int64_t)16 * 8 + fa::g_dec.n_waves) * fa::g_dec.group;
    const char* po_end = (const char*)(fa::g_dec.part_o + parts * d);
    const char* pl_end = (const char*)(fa::g_dec.part_lse + parts);
    EXPECT((const char*)fa::g_dec.part_o == lo && po_end <= lo + ws && pl_end <= lo + ws, "decode partials fit");
    check(fa_decode(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 4), P(B * 5), nullptr, 16, 64, 8, 4096, d, kvd,
                    FA_DTYPE_FP32, 0.088f, 0, P(B * 7), ws - 1, nullptr),
          FA_ERR_WORKSPACE_TOO_SMALL, "decode small workspace");
    check(fa_decode_noalloc(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 4), P(B * 5), nullptr, 16, 64, 8, 4096,
                            d, kvd, FA_DTYPE_BF16, 0.088f, 0, nullptr),
          FA_OK, "decode_noalloc valid");
  }
  check(fa_decode_noalloc(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 4), P(B * 5), nullptr, 4096, 64, 8, 1024,
                          128, kv, FA_DTYPE_BF16, 0.088f, 0, nullptr),
        FA_ERR_UNSUPPORTED, "decode_noalloc past scratch");
  check(fa_decode(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 4), P(B * 5), nullptr, 16, 64, 8, 4096, 96, kv,
                  FA_DTYPE_FP32, 0.088f, 0, P(B * 7), 1 << 30, nullptr),
        FA_ERR_UNSUPPORTED, "decode d=96");
  const int64_t ps[3] = {8 * 16 * 128, 16 * 128, 128};
  const size_t wsp = fa_decode_workspace_bytes(4, 32, 4, 64 * 16, 128, 0);
  check(fa_decode_paged(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 8), (const int32_t*)P(B * 4), P(B * 5),
                        nullptr, 4, 32, 4, 128, 300, 16, 64, ps, FA_DTYPE_BF16, 0.088f, 0, P(B * 7), wsp, nullptr),
        FA_OK, "paged valid");
  EXPECT(fa::g_dec.block_table != nullptr && fa::g_dec.page_size == 16 && fa::g_dec.max_seqlen == 1024, "paged params");
  check(fa_decode_paged(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 8), (const int32_t*)P(B * 4), P(B * 5),
                        nullptr, 4, 32, 4, 128, 300, 8, 64, ps, FA_DTYPE_BF16, 0.088f, 0, P(B * 7), wsp, nullptr),
        FA_ERR_UNSUPPORTED, "paged page 8");
  check(fa_decode_paged(P(B), P(B * 2), P(B * 3), (const int32_t*)P(B * 8), (const int32_t*)P(B * 4), P(B * 5),
                        nullptr, 4, 32, 4, 128, 300, 1 << 20, 1 << 12, ps, FA_DTYPE_BF16, 0.088f, 0, P(B * 7), wsp,
                        nullptr),
        FA_ERR_INVALID_ARGUMENT, "paged table overflow");
}

static void bwd_fp8_cases() {
  const int64_t qs[3] = {8 * 256 * 128, 256 * 128, 128}, ks[3] = {2 * 256 * 128, 256 * 128, 128};
  const size_t ws = fa_bwd_workspace_bytes(1, 8, 256);
  check(fa_bwd(P(B), P(B * 2), P(B * 3), P(B * 4), P(B * 5), (const float*)P(B * 6), P(B * 7), P(B * 8), P(B * 9), 1,
               8, 2, 256, 256, 128, qs, ks, qs, ks, FA_DTYPE_FP32, FA_DTYPE_BF16, FA_MASK_CAUSAL, 0.088f, P(B * 10), ws,
               nullptr),
        FA_OK, "bwd valid");
  check(fa_bwd(P(B), P(B * 2), P(B * 3), P(B * 4), P(B * 5), (const float*)P(B * 6), P(B), P(B * 8), P(B * 9), 1, 8, 2,
               256, 256, 128, qs, ks, qs, ks, FA_DTYPE_FP32, FA_DTYPE_BF16, FA_MASK_CAUSAL, 0.088f, P(B * 10), ws,
               nullptr),
        FA_ERR_INVALID_ARGUMENT, "bwd dq overlaps q");
  check(fa_fp8_quantize(P(B), P(B * 2), P(B * 3), nullptr, 1, 8, 2, 256, 128, qs, ks, P(B * 4), P(B * 5), P(B * 6),
                        (float*)P(B * 7), (float*)P(B * 8), (float*)P(B * 9), nullptr),
        FA_OK, "fp8 quantize valid");
  check(fa_fwd_fp8(P(B * 4), P(B * 5), P(B * 6), (const float*)P(B * 7), (const float*)P(B * 8),
                   (const float*)P(B * 9), P(B * 10), nullptr, 1, 8, 2, 256, 128, FA_DTYPE_BF16, FA_MASK_CAUSAL, 0.088f,
                   nullptr),
        FA_OK, "fp8 fwd valid");
  check(fa_fwd_fp8(P(B * 4), P(B * 5), P(B * 6), (const float*)P(B * 7), (const float*)P(B * 8),
                   (const float*)P(B * 9), P(B * 10), nullptr, 1, 8, 2, 256, 64, FA_DTYPE_BF16, FA_MASK_CAUSAL, 0.088f,
                   nullptr),
        FA_ERR_UNSUPPORTED, "fp8 fwd d=64");
}

int main() {
  for (int s = -1; s <= 6; ++s) EXPECT(fa_status_string((fa_status_t)s) != nullptr, "status string %d", s);
  fwd_cases();
  decode_cases();
  bwd_fp8_cases();
  // the error message is per thread: two threads fail differently at once
  auto worker = [](int d) {
    for (int i = 0; i < 200; ++i) {
      const int64_t s[3] = {0, 0, 0};
      fa_fwd(P(B), P(B), P(B), P(B * 2), nullptr, 1, 1, 1, 1, 1, d, s, s, s, s, FA_DTYPE_BF16, FA_DTYPE_BF16,
             FA_MASK_NONE, 1.f, nullptr);
      const char* m = fa_last_error_message();
      if (std::strstr(m, d == 96 ? "96" : "positive") == nullptr) std::abort();
    }
  };
  std::thread a(worker, 96), b(worker, 0);
  a.join();
  b.join();
  std::printf("%s: %d launcher calls, %d failures\n", g_fail ? "FAILED" : "ALL OK", fa::g_calls, g_fail);
  return g_fail ? 1 : 0;
}
