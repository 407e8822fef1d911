// Host-only check of the single kernel's launch orders (built with
// hipcc --offload-host-only; no GPU).  For each order the library builds -
// the default sequence-major order (with and without residual-mass items and
// prediction's leader items) and the early-exit position-major order - over
// a sweep of batch sizes, gamma, chunk and sampling-item counts and slot
// counts, every block number is decoded with the three decoders, and:
//   * they give the same item, whose kind, instance and part are in
//     range, and every item of every kind appears exactly once;
//   * every item a block waits for has a smaller block number.  Blocks are
//     dispatched in increasing order, so a block only ever waits for blocks
//     already running or done, and every wait ends.
// Exit status 0 = every check passed.
#include "verify_sched.h"

#include <cstdio>
#include <vector>

using namespace sv;

static int failures = 0;
static long checked = 0;
#define CHECK(c, ...)                                                  \
  do {                                                                 \
    if (!(c)) {                                                        \
      if (failures < 20) {                                             \
        std::printf("FAIL %s:%d: %s: ", __FILE__, __LINE__, #c);       \
        std::printf(__VA_ARGS__);                                      \
        std::printf("\n");                                             \
      }                                                                \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

// Block number of every item: blk[kind][instance * size + part].
struct Order {
  Sched s;
  std::vector<int64_t> blk[kKinds];
  int64_t at(int kind, int n, int part) const { return blk[kind][(size_t)n * s.size[kind] + part]; }
  int64_t max_of(int kind, int n) const {
    int64_t m = -1;
    for (int p = 0; p < s.size[kind]; ++p) m = std::max(m, at(kind, n, p));
    return m;
  }
};

static bool walk(Order& o, const char* what) {
  const Sched& s = o.s;
  CHECK(s.nseg >= 1 && s.nseg <= kMaxSeg, "%s: %d segments", what, s.nseg);
  int64_t total = 0;
  for (int k = 0; k < kKinds; ++k) {
    const int64_t n = (s.size[k] > 0 && s.count[k] > 0) ? (int64_t)s.size[k] * s.count[k] : 0;
    o.blk[k].assign((size_t)n, -1);
    total += n;
  }
  CHECK(total == s.total, "%s: %lld items listed, %lld in the order", what, (long long)total, (long long)s.total);
  if (total != s.total) return false;
  for (int64_t j = 0; j < s.total; ++j) {
    int k1, b1, p1, k2, b2, p2, k3, b3, p3;
    sched_decode_search(s, (int)j, k1, b1, p1);
    sched_decode_table(s, (int)j, k2, b2, p2);
    sched_decode_mem(s, (int)j, k3, b3, p3);
    CHECK(k1 == k2 && b1 == b2 && p1 == p2 && k1 == k3 && b1 == b3 && p1 == p3,
          "%s: block %lld: search (%d,%d,%d) table (%d,%d,%d) mem (%d,%d,%d)", what, (long long)j, k1, b1, p1,
          k2, b2, p2, k3, b3, p3);
    const bool ok = k1 >= 0 && k1 < kKinds && b1 >= 0 && b1 < s.count[k1] && p1 >= 0 && p1 < s.size[k1];
    CHECK(ok, "%s: block %lld decodes to kind %d instance %d part %d", what, (long long)j, k1, b1, p1);
    if (!ok) return false;
    int64_t& slot = o.blk[k1][(size_t)b1 * s.size[k1] + p1];
    CHECK(slot < 0, "%s: item (%d,%d,%d) at blocks %lld and %lld", what, k1, b1, p1, (long long)slot, (long long)j);
    slot = j;
    ++checked;
  }
  for (int k = 0; k < kKinds; ++k)
    for (size_t i = 0; i < o.blk[k].size(); ++i)
      CHECK(o.blk[k][i] >= 0, "%s: item kind %d index %zu never dispatched", what, k, i);
  return failures == 0;
}

#define AFTER(x, y, ...) CHECK((x) > (y), __VA_ARGS__)

// The default order: decide(b) waits for b's stream items; mass items for the
// record; sampling items for the record and (eps) every mass item; the draw
// for the record, every sampling and mass item; the final item for the
// record, target row gamma's pieces, the draw and every item that counts
// itself as a reader of the record.
static void check_default(int B, int gamma, int nc, int NM, int NB, bool pred, int slots) {
  Order o;
  o.s = make_sched(B, 2 * gamma * nc, (pred ? 2 : 1) * nc, NM, NB, slots);
  char what[160];
  std::snprintf(what, sizeof what, "default B=%d gamma=%d nc=%d NM=%d NB=%d pred=%d slots=%d", B, gamma, nc, NM,
                NB, (int)pred, slots);
  if (!walk(o, what)) return;
  for (int b = 0; b < B; ++b) {
    const int64_t dec = o.at(kItemDecide, b, 0);
    AFTER(dec, o.max_of(kItemStream, b), "%s: decide %d", what, b);
    int64_t mass_max = -1, samp_max = -1;
    for (int m = 0; m < NM; ++m) {
      AFTER(o.at(kItemMass, b, m), dec, "%s: mass %d.%d", what, b, m);
      mass_max = std::max(mass_max, o.at(kItemMass, b, m));
    }
    for (int t = 0; t < NB; ++t) {
      const int64_t x = o.at(kItemSample, b, t);
      AFTER(x, dec, "%s: sample %d.%d", what, b, t);
      AFTER(x, mass_max, "%s: sample %d.%d after mass", what, b, t);
      samp_max = std::max(samp_max, x);
    }
    const int64_t draw = o.at(kItemDraw, b, 0);
    AFTER(draw, std::max(dec, std::max(samp_max, mass_max)), "%s: draw %d", what, b);
    const int64_t fin = o.at(kItemFinal, b, 0);
    AFTER(fin, std::max(draw, o.max_of(kItemLast, b)), "%s: final %d", what, b);
  }
}

// The early-exit order: the test of (i, b) waits for the stream items of rows
// i and gamma + i of b and for the test of (i - 1, b); whichever test decides
// writes the record, so everything after waits for every test of b.
static void check_early(int B, int G, int NC, int NM, int NB, int slots) {
  Order o;
  o.s = make_sched_early(B, G, NC, NM, NB, slots);
  char what[160];
  std::snprintf(what, sizeof what, "early B=%d gamma=%d nc=%d NM=%d NB=%d slots=%d", B, G, NC, NM, NB, slots);
  if (!walk(o, what)) return;
  for (int b = 0; b < B; ++b) {
    int64_t tests = -1;
    for (int i = 0; i < G; ++i) {
      const int64_t t = o.at(kItemTest, i * B + b, 0);
      AFTER(t, o.max_of(kItemStream, i * B + b), "%s: test %d.%d", what, i, b);
      if (i > 0) AFTER(t, o.at(kItemTest, (i - 1) * B + b, 0), "%s: test %d.%d after %d", what, i, b, i - 1);
      tests = std::max(tests, t);
    }
    int64_t mass_max = -1, samp_max = -1;
    for (int m = 0; m < NM; ++m) {
      AFTER(o.at(kItemMass, b, m), tests, "%s: mass %d.%d", what, b, m);
      mass_max = std::max(mass_max, o.at(kItemMass, b, m));
    }
    for (int t = 0; t < NB; ++t) {
      const int64_t x = o.at(kItemSample, b, t);
      AFTER(x, std::max(tests, mass_max), "%s: sample %d.%d", what, b, t);
      samp_max = std::max(samp_max, x);
    }
    const int64_t draw = o.at(kItemDraw, b, 0);
    AFTER(draw, std::max(tests, std::max(samp_max, mass_max)), "%s: draw %d", what, b);
    const int64_t fin = o.at(kItemFinal, b, 0);
    AFTER(fin, std::max(draw, o.max_of(kItemLast, b)), "%s: final %d", what, b);
  }
}

int main() {
  const int Bs[] = {1, 2, 7, 64, 128, 256, 1000};
  const int gammas[] = {1, 4, 8, 63};
  const int ncs[] = {1, 4, 5, 16};
  const int slot_counts[] = {4, 64, 2048, 4096};
  for (int B : Bs)
    for (int g : gammas)
      for (int nc : ncs)
        for (int slots : slot_counts) {
          if ((int64_t)B * g * nc > 40000) continue;   // keep the sweep to seconds
          const int nts[] = {1, 19, 38};
          for (int nt : nts) {
            check_default(B, g, nc, 0, nt, false, slots);
            check_default(B, g, nc, nt, nt, false, slots);   // Saguaro with eps: mass items
            check_default(B, g, nc, 0, nt, true, slots);     // prediction: leader items
            check_early(B, g, nc, 0, nt, slots);
            check_early(B, g, nc, nt, nt, slots);
          }
        }
  std::printf("%s (%ld blocks decoded, %d failures)\n", failures ? "FAILED" : "ok", checked, failures);
  return failures ? 1 : 0;
}
