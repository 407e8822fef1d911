// Launch order of the single-kernel schedule.
#pragma once
#include "verify_sample.h"

namespace sv {

// ---------------------------------------------------------------------------
// Launch order.
//
// Step t holds, in this order: the stream items of the rows the accept tests
// read of sequence t (draft and target rows 0..gamma-1), the decision of
// sequence t - LD, the residual-mass items of t - LM (eps > 0 only), the
// sampling items of t - LB, the draw of t - LR, the stream items of target row
// gamma of t - LL and the final item of t - LF, where each exists.  The lags
// grow in that order, and LL >= B puts every target row gamma after every
// other row, so the last bytes streamed are ones no decision waits for.

//
// Early exit is position-major instead: step i*B + b holds the stream items of
// draft and target row i of sequence b, so the rows of position i+1 of a
// sequence come B steps after those of position i, and the test of (i, b)
// sits LT steps after its rows.  A test only waits for its rows and for the
// test of (i-1, b), both earlier in the order.  The sampling, draw, target
// row gamma and final items of every sequence follow the last position.

constexpr int kKinds = 8;
enum : int {
  kItemStream = 0, kItemDecide = 1, kItemMass = 2, kItemSample = 3, kItemDraw = 4, kItemLast = 5,
  kItemFinal = 6, kItemTest = 7
};

// Kind i has `count[i]` instances (sequences, or positions x sequences for
// the early-exit stream and test kinds) of `size[i]` items each, instance n at
// step lag[i] + n.  Between consecutive lag / lag + count boundaries the same
// kinds are active on every step, so the order is cut into at most
// 2 kKinds + 1 segments of equal steps; the host lists them, and a block finds
// its item with a short scan and one division on the scalar unit.
constexpr int kMaxSeg = 2 * kKinds + 1;
struct Sched {
  int lag[kKinds];
  int size[kKinds];
  int count[kKinds];
  int steps;        // max over kinds of lag + count
  int64_t total;
  int nseg;
  int seg_step[kMaxSeg];       // first step of the segment
  int seg_first[kMaxSeg];      // number of the segment's first item
  int seg_per[kMaxSeg];        // items per step (0: an empty stretch)
  unsigned seg_mask[kMaxSeg];  // kinds active on its steps
};

static int64_t sched_offset(const Sched& s, int t) {
  int64_t o = 0;
  for (int i = 0; i < kKinds; ++i) {
    int n = t - s.lag[i];
    n = n < 0 ? 0 : (n > s.count[i] ? s.count[i] : n);
    o += (int64_t)n * s.size[i];
  }
  return o;
}

// Fills steps, total and the segments from lag, size and count.
static void sched_finish(Sched& s) {
  s.steps = 0;
  for (int i = 0; i < kKinds; ++i)
    if (s.size[i] > 0 && s.count[i] > 0) s.steps = std::max(s.steps, s.lag[i] + s.count[i]);
  s.total = sched_offset(s, s.steps);
  int cut[2 * kKinds + 2];
  int nc = 0;
  cut[nc++] = 0;
  for (int i = 0; i < kKinds; ++i) {
    if (s.size[i] <= 0 || s.count[i] <= 0) continue;
    cut[nc++] = std::min(std::max(s.lag[i], 0), s.steps);
    cut[nc++] = std::min(std::max(s.lag[i] + s.count[i], 0), s.steps);
  }
  std::sort(cut, cut + nc);
  nc = (int)(std::unique(cut, cut + nc) - cut);
  s.nseg = 0;
  for (int q = 0; q < nc; ++q) {
    const int t0 = cut[q];
    if (t0 >= s.steps) break;
    unsigned mask = 0;
    int per = 0;
    for (int i = 0; i < kKinds; ++i) {
      if (s.size[i] > 0 && s.lag[i] <= t0 && t0 < s.lag[i] + s.count[i]) {
        mask |= 1u << i;
        per += s.size[i];
      }
    }
    s.seg_step[s.nseg] = t0;
    s.seg_first[s.nseg] = (int)sched_offset(s, t0);
    s.seg_per[s.nseg] = per;
    s.seg_mask[s.nseg] = mask;
    ++s.nseg;
  }
}

// NSm stream items per sequence for the rows the accept tests read, NL for
// target row gamma, NM residual-mass and NB sampling items.
static Sched make_sched(int B, int NSm, int NL, int NM, int NB, int slots) {
  Sched s;
  for (int i = 0; i < kKinds; ++i) s.count[i] = B;
  s.lag[kItemTest] = 0;
  s.size[kItemTest] = 0;
  const double spr = (double)slots / (double)(NSm + NL);   // sequences streamed per round
  auto steps = [&](int milli) { return (int)std::lround(spr * milli / 1000.0); };
  s.lag[kItemStream] = 0;
  s.lag[kItemDecide] = steps(SV_LAG_DECIDE);
  s.lag[kItemMass] = s.lag[kItemDecide] + (NM > 0 ? steps(SV_LAG_MASS) : 0);
  s.lag[kItemSample] = s.lag[kItemMass] + steps(SV_LAG_SAMPLE);
  s.lag[kItemDraw] = s.lag[kItemSample] + steps(SV_LAG_DRAW);
  s.lag[kItemLast] = std::max(B, s.lag[kItemDraw]);
  s.lag[kItemFinal] = s.lag[kItemLast] + steps(SV_LAG_FINAL);
  s.size[kItemStream] = NSm;
  s.size[kItemDecide] = 1;
  s.size[kItemMass] = NM;
  s.size[kItemSample] = NB;
  s.size[kItemDraw] = 1;
  s.size[kItemLast] = NL;
  s.size[kItemFinal] = 1;
  sched_finish(s);
  return s;
}

// Early exit: G positions, NC chunks per row.
static Sched make_sched_early(int B, int G, int NC, int NM, int NB, int slots) {
  Sched s;
  const double spr = (double)slots / (double)(2 * NC + 1);   // position-steps per round
  auto steps = [&](int milli) { return (int)std::lround(spr * milli / 1000.0); };
  for (int i = 0; i < kKinds; ++i) s.count[i] = B;
  s.count[kItemStream] = s.count[kItemTest] = G * B;
  s.lag[kItemStream] = 0;
  s.lag[kItemTest] = std::min(steps(SV_LAG_TEST), std::max(B - 1, 0));
  const int base = (G - 1) * B + s.lag[kItemTest] + 1;   // after the test of the last position
  s.lag[kItemDecide] = 0;
  s.lag[kItemMass] = base;
  s.lag[kItemSample] = base + (NM > 0 ? steps(SV_LAG_SAMPLE) : 0);
  s.lag[kItemDraw] = s.lag[kItemSample] + steps(SV_LAG_DRAW);
  s.lag[kItemLast] = std::max(G * B, s.lag[kItemDraw]);
  s.lag[kItemFinal] = s.lag[kItemLast] + steps(SV_LAG_FINAL);
  s.size[kItemStream] = 2 * NC;
  s.size[kItemTest] = 1;
  s.size[kItemDecide] = 0;
  s.size[kItemMass] = NM;
  s.size[kItemSample] = NB;
  s.size[kItemDraw] = 1;
  s.size[kItemLast] = NC;
  s.size[kItemFinal] = 1;
  sched_finish(s);
  return s;
}

// Two decoders of a block number: a binary search over the steps (the
// default order measures faster with it) and the segment table (the
// early-exit order, whose many short items gain from the shorter decode).
// Host code too, so that a host test can walk every block of an order.
__host__ __device__ inline int64_t sched_offset_dev(const Sched& s, int t) {
  int64_t o = 0;
#pragma unroll
  for (int i = 0; i < kKinds; ++i) {
    int n = t - s.lag[i];
    n = n < 0 ? 0 : (n > s.count[i] ? s.count[i] : n);
    o += (int64_t)n * s.size[i];
  }
  return o;
}
__host__ __device__ inline void sched_decode_search(const Sched& s, int j, int& kind, int& b, int& sub) {
  int lo = 0, hi = s.steps;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sched_offset_dev(s, mid) <= j) lo = mid;
    else hi = mid;
  }
  int64_t w = j - sched_offset_dev(s, lo);
  kind = kItemFinal;
  b = lo - s.lag[kItemFinal];
  sub = 0;
#pragma unroll
  for (int i = 0; i < kKinds; ++i) {
    const int bi = lo - s.lag[i];
    if (bi < 0 || bi >= s.count[i]) continue;
    if (w < s.size[i]) {
      kind = i;
      b = bi;
      sub = (int)w;
      return;
    }
    w -= s.size[i];
  }
}
// The segment of block j by a binary search over the segments' first items,
// then the kinds of its steps: every index is dynamic, so `s` must be memory
// the scalar unit reads directly (the kernel argument segment, see
// FusedArgs) - a few dependent scalar loads instead of the whole table held
// in scalar registers.
__host__ __device__ inline void sched_decode_mem(const Sched& s, int j, int& kind, int& b, int& sub) {
  int lo = 0, hi = s.nseg;   // the last segment starting at or before j (an empty
  while (hi - lo > 1) {      // one shares its start with the next)
    const int mid = (lo + hi) >> 1;
    if (s.seg_first[mid] <= j) lo = mid;
    else hi = mid;
  }
  const int per = s.seg_per[lo];
  const unsigned mask = s.seg_mask[lo];
  const int rel = j - s.seg_first[lo];
  const int dt = rel / per;
  const int t = s.seg_step[lo] + dt;
  int w = rel - dt * per;
  kind = kItemFinal;
  b = 0;
  sub = 0;
  for (int i = 0; i < kKinds; ++i) {
    if ((mask >> i) & 1u) {
      const int size = s.size[i];
      if (w < size) {
        kind = i;
        b = t - s.lag[i];
        sub = w;
        return;
      }
      w -= size;
    }
  }
}
// Every index into the table is a constant (unrolled loops and selects), so
// the table is read straight from the kernel arguments.
__host__ __device__ inline void sched_decode_table(const Sched& s, int j, int& kind, int& b, int& sub) {
  int step = s.seg_step[0], first = s.seg_first[0], per = s.seg_per[0];
  unsigned mask = s.seg_mask[0];
#pragma unroll
  for (int i = 1; i < kMaxSeg; ++i) {   // the last segment starting at or before j (empty
    if (i < s.nseg && s.seg_first[i] <= j) {   // ones share their start with the next)
      step = s.seg_step[i];
      first = s.seg_first[i];
      per = s.seg_per[i];
      mask = s.seg_mask[i];
    }
  }
  const int rel = j - first;
  const int dt = rel / per;
  const int t = step + dt;
  int w = rel - dt * per;
  kind = kItemFinal;
  b = 0;
  sub = 0;
  bool found = false;
#pragma unroll
  for (int i = 0; i < kKinds; ++i) {
    if (!found && ((mask >> i) & 1u)) {
      if (w < s.size[i]) {
        kind = i;
        b = t - s.lag[i];
        sub = w;
        found = true;
      } else {
        w -= s.size[i];
      }
    }
  }
}

}  // namespace sv
