// Host-side checks of the library's C entry points, built host-only with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code (no GPU,
// no kernel launch): the workspace-size queries over a sweep of sizes,
// including sizes at the limits of int, and every entry point's rejection of
// bad arguments.  Any sanitizer report, or a check that fails, ends the
// program with a non-zero status.
#include "spec_verify.h"

#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>

static int failures = 0;
#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                              \
    }                                                          \
  } while (0)

// Never dereferenced: every call below fails validation before any use.
static void* const F = reinterpret_cast<void*>(4096);
#define FI reinterpret_cast<int32_t*>(F)
#define FF reinterpret_cast<float*>(F)
#define FU reinterpret_cast<uint64_t*>(F)

static int verify(int B, int g, int V, float T, int dtype, const void* d, const void* ws,
                  size_t wsb) {
  return spec_verify(d, F, dtype, FI, FF, FF, B, g, V, T, nullptr, FI, FI, nullptr, nullptr,
                     nullptr, nullptr, const_cast<void*>(ws), wsb, nullptr);
}

static void size_queries() {
  const int Bs[] = {-1, 0, 1, 7, 256, 65536, INT_MAX};
  const int gs[] = {-1, 0, 1, 8, 63, 64, INT_MAX};
  const int Vs[] = {-1, 0, 1, 7, 152064, 1 << 24, INT_MAX};
  for (int B : Bs)
    for (int g : gs)
      for (int V : Vs)
        for (int dt = -1; dt <= 2; ++dt) {
          const size_t w = spec_workspace_bytes(B, g, V, dt);
          const size_t p = spec_predict_workspace_bytes(B, g, V, dt);
          const size_t gr = spec_greedy_workspace_bytes(B, g, V, dt);
          const bool ok = B >= 0 && g >= 1 && g <= 63 && V >= 1 && (dt == SPEC_F32 || dt == SPEC_BF16);
          if (!ok) {
            CHECK(w == 0);
          }
          if (ok && B > 0 && w != 0) {
            // a size that is reported covers at least one 32-bit word per row pair
            CHECK(w >= (size_t)B * (size_t)g);
          }
          (void)p;
          (void)gr;
        }
}

static void rejections() {
  // spec_verify / spec_verify_saguaro
  CHECK(verify(-1, 3, 100, 1.0f, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 0, 100, 1.0f, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 64, 100, 1.0f, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 3, 0, 1.0f, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 3, 100, 0.0f, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 3, 100, -1.0f, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 3, 100, NAN, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 3, 100, INFINITY, SPEC_BF16, F, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 3, 100, 1.0f, 7, F, F, 1u << 30) == SPEC_EDTYPE);
  CHECK(verify(4, 3, 100, 1.0f, SPEC_BF16, nullptr, F, 1u << 30) == SPEC_EINVAL);
  CHECK(verify(4, 3, 100, 1.0f, SPEC_BF16, F, nullptr, 1u << 30) == SPEC_EWORKSPACE);
  CHECK(verify(4, 3, 100, 1.0f, SPEC_BF16, F, F, 8) == SPEC_EWORKSPACE);
  CHECK(verify(0, 3, 100, 1.0f, SPEC_BF16, nullptr, nullptr, 0) == SPEC_OK);
  CHECK(verify(INT_MAX, 63, INT_MAX, 1.0f, SPEC_BF16, F, F, 1u << 30) != SPEC_OK);
  CHECK(spec_verify_saguaro(F, F, SPEC_BF16, FI, FF, FF, 4, 3, 100, 1.0f, nullptr, FI, FI, nullptr,
                            nullptr, nullptr, nullptr, F, 1u << 30, nullptr, -1.0f) == SPEC_EINVAL);
  CHECK(spec_verify_saguaro(F, F, SPEC_BF16, FI, FF, FF, 4, 3, 100, 1.0f, nullptr, FI, FI, nullptr,
                            nullptr, nullptr, nullptr, F, 1u << 30, nullptr, NAN) == SPEC_EINVAL);
  // spec_verify_early
  CHECK(spec_verify_early(F, F, SPEC_BF16, FI, FF, FF, 4, 64, 100, 1.0f, nullptr, FI, FI, nullptr,
                          nullptr, nullptr, nullptr, 0, 0.0f, F, 1u << 30, nullptr) == SPEC_EINVAL);
  // spec_verify_ex: bad top-p, bad eps
  spec_options o = {0, 0.0f, 0, nullptr, nullptr, nullptr, nullptr, 1.5f};
  CHECK(spec_verify_ex(F, F, SPEC_BF16, FI, FF, FF, 4, 3, 100, 1.0f, nullptr, FI, FI, nullptr,
                       nullptr, nullptr, nullptr, &o, F, 1u << 30, nullptr) == SPEC_EINVAL);
  o.top_p = NAN;
  CHECK(spec_verify_ex(F, F, SPEC_BF16, FI, FF, FF, 4, 3, 100, 1.0f, nullptr, FI, FI, nullptr,
                       nullptr, nullptr, nullptr, &o, F, 1u << 30, nullptr) == SPEC_EINVAL);
  o.top_p = 0.0f;
  o.saguaro = 1;
  o.eps = -1.0f;
  CHECK(spec_verify_ex(F, F, SPEC_BF16, FI, FF, FF, 4, 3, 100, 1.0f, nullptr, FI, FI, nullptr,
                       nullptr, nullptr, nullptr, &o, F, 1u << 30, nullptr) == SPEC_EINVAL);
  // spec_verify_predict: cand required
  CHECK(spec_verify_predict(F, F, SPEC_BF16, FI, FF, FF, 4, 3, 100, 1.0f, nullptr, FI, FI, nullptr,
                            nullptr, nullptr, nullptr, 0, 0.0f, nullptr, nullptr, nullptr, F,
                            1u << 30, nullptr) == SPEC_EINVAL);
  // spec_predict_outcomes
  CHECK(spec_predict_outcomes(F, SPEC_BF16, -1, 3, 100, nullptr, nullptr, FI, nullptr, nullptr, F,
                              1u << 30, nullptr) == SPEC_EINVAL);
  CHECK(spec_predict_outcomes(F, 9, 4, 3, 100, nullptr, nullptr, FI, nullptr, nullptr, F, 1u << 30,
                              nullptr) == SPEC_EDTYPE);
  CHECK(spec_predict_outcomes(F, SPEC_BF16, 4, 3, 100, FI, nullptr, FI, nullptr, nullptr, F,
                              1u << 30, nullptr) == SPEC_EINVAL);
  CHECK(spec_predict_outcomes(F, SPEC_BF16, 4, 3, 100, nullptr, nullptr, FI, nullptr, nullptr, F, 8,
                              nullptr) == SPEC_EWORKSPACE);
  // spec_verify_greedy
  CHECK(spec_verify_greedy(F, SPEC_BF16, FI, 4, 64, 100, nullptr, FI, FI, nullptr, nullptr, nullptr,
                           F, 1u << 30, nullptr) == SPEC_EINVAL);
  CHECK(spec_verify_greedy(nullptr, SPEC_BF16, FI, 4, 3, 100, nullptr, FI, FI, nullptr, nullptr,
                           nullptr, F, 1u << 30, nullptr) == SPEC_EINVAL);
  // spec_verify_noalloc: beyond its static scratch, bad dtype, bad gamma
  CHECK(spec_verify_noalloc(F, F, SPEC_BF16, FI, FF, FF, 512, 8, 152064, 1.0f, nullptr, FI, FI,
                            nullptr, nullptr, nullptr, nullptr, nullptr) == SPEC_ESCRATCH);
  CHECK(spec_verify_noalloc(F, F, 5, FI, FF, FF, 4, 3, 100, 1.0f, nullptr, FI, FI, nullptr, nullptr,
                            nullptr, nullptr, nullptr) == SPEC_EDTYPE);
  CHECK(spec_verify_noalloc(F, F, SPEC_BF16, FI, FF, FF, 4, 64, 100, 1.0f, nullptr, FI, FI, nullptr,
                            nullptr, nullptr, nullptr, nullptr) == SPEC_EINVAL);
  // pipeline helpers
  CHECK(spec_synthetic_busy(-1, nullptr, 0, nullptr) == SPEC_EINVAL);
  CHECK(spec_synthetic_busy(1000, nullptr, 3, nullptr) == SPEC_EINVAL);
  CHECK(spec_synth_draft(F, SPEC_BF16, 100, 0, FF, 8, 4, 3, FI, nullptr, FI, nullptr) == SPEC_EINVAL);
  CHECK(spec_synth_draft(F, SPEC_BF16, 100, 10, FF, 8, 4, 0, nullptr, nullptr, nullptr, nullptr) ==
        SPEC_OK);
  CHECK(spec_synth_rows(F, SPEC_BF16, 100, 10, 64, 2, FI, FI, F, nullptr) == SPEC_EINVAL);
  CHECK(spec_ssd_prespeculate(F, SPEC_BF16, 100, 10, FF, 0, 4, 2, FI, nullptr, FI, nullptr) ==
        SPEC_EINVAL);
  CHECK(spec_ssd_advance(F, SPEC_BF16, 100, 10, FF, 8, 4, 2, FI, FI, FI, FI, nullptr, nullptr, FI,
                         FI, FI, nullptr) == SPEC_EINVAL);
  CHECK(spec_read_bandwidth(nullptr, 1024, FU, nullptr) == SPEC_EINVAL);
  for (int s = -10; s <= 5; ++s) CHECK(spec_status_str(s) != nullptr);
}

int main() {
  size_queries();
  rejections();
  std::printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
