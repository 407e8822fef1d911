// Arguments, hand-off slots and shared helpers of the verification kernels.
#pragma once
#include "common.h"
#include "predict.h"
#include "spec_verify.h"

#include <cmath>
#include <limits.h>
#include <algorithm>
#include <type_traits>

#undef SV_FILE
#define SV_FILE 1

namespace sv {

enum : int { kModeTarget = 0, kModeResidual = 1, kModeSaguaro = 2, kModeSaguaroEps = 3 };

#ifndef SV_TILES_PER_ITEM
#define SV_TILES_PER_ITEM 4
#endif
#ifndef SV_STREAM_UNROLL
#define SV_STREAM_UNROLL 4
#endif
// 1: every item in one kernel (the default); 0: one kernel per item kind.
#ifndef SV_FUSED
#define SV_FUSED 1
#endif
// Lags of the decision, residual-mass, sampling, draw and final items behind
// their sequence's stream items, in thousandths of a round (one round = as
// many stream items as the GPU holds at once); each is added to the one
// before (the final item's to the lag of target row gamma).
#ifndef SV_LAG_DECIDE
#define SV_LAG_DECIDE 1400
#endif
#ifndef SV_LAG_MASS
#define SV_LAG_MASS 1000
#endif
#ifndef SV_LAG_SAMPLE
#define SV_LAG_SAMPLE 1000
#endif
#ifndef SV_LAG_DRAW
#define SV_LAG_DRAW 800
#endif
#ifndef SV_LAG_FINAL
#define SV_LAG_FINAL 200
#endif
// Early exit: lag of a position's test behind its rows (thousandths of a round).
#ifndef SV_LAG_TEST
#define SV_LAG_TEST 800
#endif
// Early exit: stream chunk length (a multiple of the default; fewer, longer
// items per row make the items that skip rows fewer).
#ifndef SV_EARLY_CHUNK
#define SV_EARLY_CHUNK SV_CHUNK
#endif
#ifndef SV_SAMPLE_NT
#define SV_SAMPLE_NT 0
#endif
constexpr int kTilesPerItem = SV_TILES_PER_ITEM;
constexpr int kShortTiles = kTilesPerItem >= 2 ? kTilesPerItem / 2 : 1;   // short calls' sampling items
constexpr bool kSampleNT = SV_SAMPLE_NT != 0;   // nontemporal loads in the sampling items
// The shortest chunk (one batch stride), and the stream items below which a
// call shortens its chunks towards it.
constexpr int kMinChunk = SV_STREAM_UNROLL * kThreads * kUnit;
constexpr int64_t kSmallCallItems = 512;
static_assert(kChunk % kMinChunk == 0 && (kChunk / kMinChunk & (kChunk / kMinChunk - 1)) == 0,
              "chunks halve down to the batch stride");
// The shortest chunk of a small call (its chunks halve down to it): one tile.
#ifndef SV_SMALL_CHUNK
#define SV_SMALL_CHUNK 2048
#endif
constexpr int kSmallChunk = SV_SMALL_CHUNK;
static_assert(kSmallChunk % kTile == 0 && kChunk % kSmallChunk == 0 &&
                  (kChunk / kSmallChunk & (kChunk / kSmallChunk - 1)) == 0,
              "small-call chunks are whole tiles and halve down from the default chunk");
static_assert(kChunk % (SV_STREAM_UNROLL * kThreads * kUnit) == 0,
              "a stream chunk must hold whole batches");
constexpr unsigned kMaxPolls = 1u << 22;   // bounded waits: about a quarter of a second

// ---------------------------------------------------------------------------
// Slots.

__device__ __forceinline__ uint64_t slot_word(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  if (b == ~0ull) b = 0x7FF8000000000000ull;   // keep the empty word 0 unreachable
  return ~b;
}
__device__ __forceinline__ double slot_value(uint64_t w) { return __longlong_as_double((long long)~w); }
__device__ __forceinline__ void slot_put(uint64_t* p, double x) { st_dev_u64(p, slot_word(x)); }
__device__ __forceinline__ void slot_clear(uint64_t* p) { st_dev_u64(p, 0ull); }
__device__ __forceinline__ void slot_put32(unsigned* p, float x) {
  uint32_t b = __float_as_uint(x);
  if (b == ~0u) b = 0x7FC00000u;
  __hip_atomic_store(p, ~b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void slot_clear32(unsigned* p) {
  __hip_atomic_store(p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A sequence's decision, written by its decision item.  Each 64-bit word is
// stored as its complement (no word of a record is all ones), so a word is 0
// until written, and readers poll the words themselves.
struct SeqRec {
  uint64_t mask;
  int k;
  int valid;
  int mode;         // weights of the draw
  float Mt;         // integer offset of the row drawn from (target row k)
  float K_hi, K_lo; // log2(p_j/q_j) = (ld_j - lt_j) * c_T + K
  double Zt;        // sum_j 2^(lt_j c_T - Mt) over target row k
};
static_assert(sizeof(SeqRec) % 8 == 0, "SeqRec is moved as 64-bit words");
constexpr int kRecWords = sizeof(SeqRec) / 8;

__device__ __forceinline__ void store_rec(SeqRec* p, const SeqRec& r) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(&r);
#pragma unroll
  for (int i = 0; i < kRecWords; ++i) st_dev_u64(reinterpret_cast<uint64_t*>(p) + i, ~w[i]);
}
__device__ __forceinline__ void clear_rec(SeqRec* p) {
#pragma unroll
  for (int i = 0; i < kRecWords; ++i) st_dev_u64(reinterpret_cast<uint64_t*>(p) + i, 0ull);
}

// One 128-byte line per sequence: [0] = residual-mass and sampling items that
// have read the decision record; [2..3] the drawn token's slot.  Early exit
// also uses [4] = 64 - (a position known to stop the sequence), raised by
// atomic max (0: none known), [5] = positions known accepted in a row from
// position 0, [6] = position tests done.
constexpr int kFlagStride = 32;
constexpr int kStopWord = 4, kProgWord = 5, kTestsWord = 6;
// A stream item of early exit that finds its position beyond a known stop
// publishes these instead of its piece (their values are NaN; no real piece
// has these words).
constexpr uint64_t kSkipPiece = 1ull;
constexpr unsigned kSkipRaw = 1u;

// Top-p state of one row (the rows of the rule, numbered as the pieces):
// its normaliser, the radix selection of the nucleus threshold, and the
// result.  Masses are in units of 2^M (the row's integer offset).
struct TopPRow {
  double M, Z;       // the row's offset and normaliser
  double rem;        // mass still to reach inside the selected key prefix
  double above;      // mass of the keys above the selected prefix
  double P;          // nucleus mass / Z (1 without a cut)
  uint32_t prefix;   // selected high digits of the threshold key
  float L;           // threshold logit: the nucleus is l >= L (-inf: no cut)
};
constexpr int kDigits = 256;   // 8-bit radix digits

struct VerifyArgs {
  const void* draft;
  const void* target;
  const int32_t* tokens;
  const float* u_acc;
  const float* u_smp;
  const int32_t* in_len;
  int32_t* out_tokens;
  int32_t* out_acc;
  int32_t* out_first_reject;
  uint64_t* out_mask;
  int32_t* out_len;
  spec_diag diag;
  unsigned* err;     // nonzero once a bounded wait timed out
  uint64_t* part;    // [B][2*gamma+1][nc] slots: chunk log2-normalisers
  unsigned* mraw;    // [B][2*gamma+1][nc] 32-bit slots: chunk maxima of the raw logits
  SeqRec* seq;       // [B]
  unsigned* flag;    // [B * kFlagStride]: record read counts
  uint64_t* tiles;   // [B][ntile] slots: tile sums of the sampling weights
  uint64_t* mass;    // [B][nt] slots: residual sums of the residual-mass items (eps > 0)
  uint64_t* rsum;    // [B][nt] slots: residual sums of the sampling items (Saguaro)
  Top3* cpart;       // [B][gamma+1][nc] lane leaders of the draft rows (outcome prediction)
  uint64_t* ref;     // [B][ntile][4] slots: fp64 tile sums of a refined residual draw
  int refine;        // 1: small residual masses are refined (by the final items)
  int B, gamma, V;
  int nc, chunk;     // stream chunks per row and their length
  int ntile, nt;     // sampling tiles per row; sampling items per sequence
  float c_hi, c_lo;  // log2(e) / T as an unevaluated float pair, c_lo > 0
  double cTd;        // c_hi + c_lo
  double invT;
  int saguaro;
  float eps;
  int early;         // early exit: rows beyond the first rejection are not needed
  const float* temps;   // [B] per-sequence temperatures, or NULL (c_hi, c_lo, cTd, invT for all)
  TopPRow* topp;        // [B][2*gamma+1] with a top-p cut, else NULL
  double* hist;         // [B][2*gamma+1][kDigits] radix histograms of the cut
  unsigned* redo;       // [2 + B*(2*gamma+1)]: rows the counting kernel leaves to the in-place
                        // finish (count, work-groups done, then row + 1 each, with a flag
                        // where the row's counters wrapped)
  float top_p;
#if SV_CHECKS
  unsigned* chk;        // the workspace's second word: site of the first failed check
  // Elements of each array (diag arrays: B rows of their width).
  int64_t n_part, n_mraw, n_seq, n_flag, n_tiles, n_mass, n_rsum, n_cpart, n_ref, n_topp, n_hist,
      n_redo, n_tokens, n_u_acc, n_u_smp, n_in_len, n_temps, n_out_tokens, n_out_acc,
      n_out_first_reject, n_out_mask, n_out_len;
#endif
};

// The temperature scale of sequence b: log2(e) / T as an unevaluated float
// pair (c_hi rounded toward zero, so c_lo > 0), their double sum, and 1 / T.
// Per-sequence temperatures are scaled here exactly as the host scales the
// common one; a temperature that is not finite and positive is scaled as 1
// and makes the sequence invalid (decision items check temp_ok).
struct TCoef {
  float c_hi, c_lo;
  double cTd, invT;
};
__device__ __forceinline__ bool temp_ok(float T) { return T > 0.f && T <= 3.402823466e38f; }
__device__ __forceinline__ float seq_temp(const VerifyArgs& a, int b) {
  return a.temps ? uni(*SV_AT(a, temps, b)) : 1.f;
}
__device__ __forceinline__ TCoef temp_coef(const VerifyArgs& a, int b) {
  TCoef t;
  if (!a.temps) {
    t.c_hi = a.c_hi;
    t.c_lo = a.c_lo;
    t.cTd = a.cTd;
    t.invT = a.invT;
    return t;
  }
  float T = seq_temp(a, b);
  if (!temp_ok(T)) T = 1.f;
  const double c = 1.4426950408889634073599246810019 / (double)T;
  float ch = (float)c;
  if ((double)ch >= c) ch = __int_as_float(__float_as_int(ch) - 1);   // next float toward zero
  float cl = (float)(c - (double)ch);
  if (!(cl > 0.f)) cl = 1.17549435e-38f;
  t.c_hi = uni(ch);
  t.c_lo = uni(cl);
  t.cTd = uni((double)t.c_hi + (double)t.c_lo);
  t.invT = uni(1.0 / (double)T);
  return t;
}

template <int DT>
__device__ __forceinline__ const void* row_ptr(const VerifyArgs& a, int b, int r) {
  // r < gamma: draft row r; otherwise target row r - gamma.  The base is
  // chosen by integer arithmetic: a select between the two argument fields
  // can be turned into a load from a selected field address, which keeps
  // the kernel's arguments in scratch memory.
  const int64_t es = DT == kBF16 ? 2 : 4;
#if SV_CHECKS
  b = (int)SV_IDX(a, b, a.B);
  r = (int)SV_IDX(a, r, 2 * a.gamma + 1);
#endif
  const bool is_draft = r < a.gamma;
  const int64_t idx = (int64_t)b * (a.gamma + 1) + (is_draft ? r : r - a.gamma);
  const uintptr_t t = reinterpret_cast<uintptr_t>(a.target);
  const uintptr_t base = t + (is_draft ? reinterpret_cast<uintptr_t>(a.draft) - t : (uintptr_t)0);
  return reinterpret_cast<const char*>(base) + idx * a.V * es;
}

// Bounded polls.  A timeout (or an error already recorded by another
// work-group) records the error and gives up.
__device__ __forceinline__ bool give_up(const VerifyArgs& a, unsigned& polls) {
  ++polls;
  if ((polls & 63u) == 0u &&
      (polls > kMaxPolls || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
    __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
  __builtin_amdgcn_s_sleep(2);
  return false;
}
__device__ __forceinline__ unsigned ld_dev_u32(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The slot's word once it is written, or 0 if the wait gave up (a value
// read from 0 is NaN, see slot_value; callers that derive an index or a
// token from the word check for 0 first).
__device__ __forceinline__ uint64_t poll(const VerifyArgs& a, const uint64_t* p) {
  uint64_t w = ld_dev_u64(p);
  unsigned polls = 0;
  while (w == 0ull && !give_up(a, polls)) w = ld_dev_u64(p);
  return w;
}

// Decode a decision record from the words as read (each stored as its
// complement, so 0 = not written).  If any word is missing - its wait gave
// up - the record is "lost": it decodes as an invalid sequence with k = 0
// and the target mode, so no index or mode is ever taken from an unwritten
// word, and `lost` tells the final item to report the sequence invalid.
__host__ __device__ inline SeqRec decode_rec(const uint64_t (&raw)[kRecWords], bool& lost) {
  lost = false;
  for (int i = 0; i < kRecWords; ++i) lost = lost || raw[i] == 0ull;
  SeqRec r;
  if (lost) {
    r.mask = 0ull;
    r.k = 0;
    r.valid = 0;
    r.mode = kModeTarget;
    r.Mt = 0.f;
    r.K_hi = r.K_lo = 0.f;
    r.Zt = 1.0;
    return r;
  }
  uint64_t w[kRecWords];
  for (int i = 0; i < kRecWords; ++i) w[i] = ~raw[i];
  static_assert(sizeof(w) == sizeof(SeqRec), "a record is its words");
  __builtin_memcpy(&r, w, sizeof(r));
  return r;
}

// The sequence's decision record: thread 0 waits for each word, the
// work-group reads it from LDS (COUNT: thread 0 then counts this item as done
// with the record).  The fields end up in scalar registers.  `lost`: the
// wait gave up (see decode_rec).
template <bool COUNT>
__device__ __forceinline__ SeqRec wait_rec(const VerifyArgs& a, int b, bool& lost) {
  __shared__ uint64_t w[kRecWords];
  if (threadIdx.x == 0) {
    // All words are requested together, again until every one has arrived.
    const uint64_t* p = reinterpret_cast<const uint64_t*>(SV_AT(a, seq, b));
    uint64_t v[kRecWords];
#pragma unroll
    for (int i = 0; i < kRecWords; ++i) v[i] = ld_dev_u64(p + i);
    unsigned polls = 0;
    for (;;) {
      bool all = true;
#pragma unroll
      for (int i = 0; i < kRecWords; ++i) all = all && v[i] != 0ull;
      if (all || give_up(a, polls)) break;
#pragma unroll
      for (int i = 0; i < kRecWords; ++i)
        if (v[i] == 0ull) v[i] = ld_dev_u64(p + i);
    }
#pragma unroll
    for (int i = 0; i < kRecWords; ++i) w[i] = v[i];
  }
  __syncthreads();
  uint64_t raw[kRecWords];
#pragma unroll
  for (int i = 0; i < kRecWords; ++i) raw[i] = uni(w[i]);
  SeqRec r = decode_rec(raw, lost);
  if (COUNT) {
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(SV_AT(a, flag, (int64_t)b * kFlagStride), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
  return r;
}
template <bool COUNT>
__device__ __forceinline__ SeqRec wait_rec(const VerifyArgs& a, int b) {
  bool lost;
  return wait_rec<COUNT>(a, b, lost);
}

}  // namespace sv
