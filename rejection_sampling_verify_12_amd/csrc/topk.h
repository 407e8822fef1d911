// Top-3 of draft logits for outcome prediction ("Speculative Speculative
// Decoding (Saguaro)", section 3.1: the bonus token of each outcome is
// predicted from the draft logits' top-3).  Shared by the stand-alone
// prediction kernels and the verification kernel that ranks draft rows while
// streaming them.
//
// Order: larger logit first, equal logits by lower token id, +0.0 == -0.0.
// Elements are compared as 64-bit keys: an order-preserving map of the
// float's bits above the complemented index, so key order is that order and
// 0 never occurs for a real element.
#pragma once
#include "common.h"

namespace sv {

// One chunk's contribution for one row.
struct Top3 {
  uint64_t key[3];   // descending; 0 = none
  uint64_t nan;      // nonzero when the chunk held a NaN
};

__device__ __forceinline__ uint64_t make_key(uint32_t bits, int64_t idx) {
  if (bits == 0x80000000u) bits = 0u;
  const uint32_t mono = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  return ((uint64_t)mono << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}
__device__ __forceinline__ int key_index(uint64_t k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu));
}

__device__ __forceinline__ void insert3(uint64_t (&t)[3], uint64_t k) {
  if (k > t[2]) {
    if (k > t[1]) {
      t[2] = t[1];
      if (k > t[0]) {
        t[1] = t[0];
        t[0] = k;
      } else {
        t[1] = k;
      }
    } else {
      t[2] = k;
    }
  }
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t t = __shfl_xor(v, o, 64);
    v = t > v ? t : v;
  }
  return v;
}

// The wave's three largest keys (every lane gets them).  Each lane offers a
// descending list of up to three distinct keys; keys are unique across
// lanes, so the lane that owns a winner drops it before the next round.
__device__ __forceinline__ void wave_top3(uint64_t (&t)[3], uint64_t (&out)[3]) {
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    out[r] = wave_max_u64(t[0]);
    if (out[r] != 0 && t[0] == out[r]) {
      t[0] = t[1];
      t[1] = t[2];
      t[2] = 0;
    }
  }
}

// Lane leaders.  A lane that streams units j, j + kTile, j + 2 kTile, ... of a
// chunk keeps only its largest logit and the start index of the first unit
// holding it.  Ranked by (logit, that unit's index), the three best lanes of a
// row hold the row's top-3: a lane holding a top-3 element has its own best
// element at least as high in the order, and at most two other lanes can
// have a best element above that element.  Within a lane the unit index
// orders its best element correctly against other lanes' (unit starts are
// multiples of eight and each lane's units are disjoint).
//
// One batch of N units of eight values (unit u starts at index jb + u kTile,
// um[u] its maximum, bm the batch's): update the lane's best unit (pos < 0
// before the first one).  mx is the lane's maximum before the batch; the
// caller raises it afterwards.
template <int N>
__device__ __forceinline__ void lead_batch(const float (&um)[N], float bm, int jb, float& mx,
                                           int& pos) {
  if (pos < 0 || bm > mx) {
    int q = N - 1;
#pragma unroll
    for (int u = N - 2; u >= 0; --u)
      if (um[u] == bm) q = u;
    pos = jb + q * kTile;
  }
}

}  // namespace sv
