// Host-only check of the decision-record decode (built with
// hipcc --offload-host-only; no GPU): a record whose words did not all arrive
// - a bounded wait that gave up - decodes as "lost": an invalid sequence with
// k = 0 and the target mode, so no item derives a row index, a uniform index
// or a weight mode from an unwritten word; a complete record decodes to the
// values stored.  Exit status 0 = every check passed.
#include "verify_args.h"

#include <cstdio>
#include <cstring>

using sv::SeqRec;
using sv::kRecWords;

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);     \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static void stored_words(const SeqRec& r, uint64_t (&raw)[kRecWords]) {
  uint64_t w[kRecWords];
  std::memcpy(w, &r, sizeof(r));
  for (int i = 0; i < kRecWords; ++i) raw[i] = ~w[i];   // as store_rec writes them
}

static void check_lost(const uint64_t (&raw)[kRecWords], int gamma) {
  bool lost = false;
  const SeqRec r = sv::decode_rec(raw, lost);
  CHECK(lost);
  CHECK(r.valid == 0);
  CHECK(r.k == 0);
  CHECK(r.mode == sv::kModeTarget);
  CHECK(r.mask == 0ull);
  // The indices an item would form from k stay inside the row and uniform arrays.
  CHECK(r.k >= 0 && r.k <= gamma);
}

int main() {
  const int gamma = 8;
  // Nothing arrived: every word still 0 (the old decode read each as ~0).
  uint64_t none[kRecWords] = {};
  check_lost(none, gamma);
  // A complete record, then every pattern of missing words.
  SeqRec r;
  std::memset(&r, 0, sizeof(r));
  r.mask = 0x5ull;
  r.k = 3;
  r.valid = 1;
  r.mode = sv::kModeResidual;
  r.Mt = 12.f;
  r.K_hi = -0.25f;
  r.K_lo = 1e-9f;
  r.Zt = 3.5;
  uint64_t raw[kRecWords];
  stored_words(r, raw);
  bool lost = true;
  const SeqRec d = sv::decode_rec(raw, lost);
  CHECK(!lost);
  CHECK(std::memcmp(&d, &r, sizeof(r)) == 0);
  for (unsigned m = 1; m < (1u << kRecWords); ++m) {
    uint64_t part[kRecWords];
    for (int i = 0; i < kRecWords; ++i) part[i] = (m >> i) & 1u ? 0ull : raw[i];
    check_lost(part, gamma);
  }
  // An invalid sequence's record (written by its decision item) is not lost.
  SeqRec inv = r;
  inv.valid = 0;
  inv.k = gamma;
  inv.mode = sv::kModeTarget;
  stored_words(inv, raw);
  const SeqRec di = sv::decode_rec(raw, lost);
  CHECK(!lost && di.valid == 0 && di.k == gamma);
  std::printf("%s: %d failure(s)\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
