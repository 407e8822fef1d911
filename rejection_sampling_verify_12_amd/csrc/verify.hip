// Batched speculative-sampling verification for gfx950.
//
// The rule is the one of "Speculative Decoding: small model guesses, large
// model verifies" (section 3: accept x iff u < min(1, q(x)/p(x)), stop at the
// first rejection, resample from (q-p)+ / sum(q-p)+; section 2: the bonus
// after gamma acceptances comes from the target's position gamma), with the
// Saguaro resampling option of "Speculative Speculative Decoding (Saguaro)"
// (section 3.2: proportional to sqrt(p_D * p_residual)).
//
// Work items (each one 256-thread work-group's job):
//   stream (b, r, c): stream chunk c of row r of sequence b once from HBM and
//     reduce it to a piece of the row's tempered-softmax log-normaliser,
//     v = log2 sum_j 2^(l_j c_T), c_T = log2(e) / T.  c_T is an unevaluated
//     float pair (two FMAs per logit) so the temperature is exact; each lane
//     keeps an integer offset, so every rescale is an exact ldexp, tree-sums
//     each batch of its logits in fp32 and accumulates in fp64.
//   decide (b): merge the pieces of the rows the accept tests read (fp64),
//     run the accept test at every draft position (fp64, wave ballot -> first
//     rejection k) and write the sequence's decision record.
//   residual mass (b, s), Saguaro with eps > 0 only: the residual weight sum
//     over a few 2048-logit tiles of row pair k, which the eps clamp needs.
//   sample (b, s): per-tile sums of the sampling weights over a few tiles of
//     row pair k, or of target row gamma after a full acceptance (the bonus
//     draw, each tile with its own offset, so it needs no row normaliser).
//   draw (b): locate the tile holding u * total (fp64 scan over the tile
//     sums, token order) and rescan it (fp64 prefix over the same per-lane
//     fp32 sums): the drawn token.
//   final (b): check target row gamma (read by the bonus draw only, hence
//     streamed last) and write the outputs.
//
// Hand-off between work-groups uses 64-bit slots that are 0 when empty: a
// producer stores ~bits(value) with one device-coherent store, a consumer
// polls (bounded) until the slot is nonzero and clears it after use, so the
// workspace is all zero again when a call ends.  No item waits for anything
// but items of the same sequence that come earlier in the launch order.
//
// Default launch: one kernel whose blocks run the items in steps (see the
// launch order below): the stream items of sequence t, then the later items
// of earlier sequences, so that a sequence's decision, sampling and draw run
// while other sequences stream; the target rows gamma, which no decision
// waits for, come last.  Work-groups are dispatched in block order, so the
// smallest unfinished block has every item it waits for finished and can
// always run; a wait that still times out sets the error word and gives up
// instead of hanging.
#include "common.h"
#include "predict.h"
#include "spec_verify.h"

#include <cmath>
#include <limits.h>
#include <algorithm>
#include <type_traits>

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
constexpr bool kSampleNT = SV_SAMPLE_NT != 0;   // nontemporal loads in the sampling items
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
  float top_p;
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
  return a.temps ? uni(a.temps[b]) : 1.f;
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
  // r < gamma: draft row r; otherwise target row r - gamma.
  const int64_t es = DT == kBF16 ? 2 : 4;
  const bool is_draft = r < a.gamma;
  const int64_t idx = (int64_t)b * (a.gamma + 1) + (is_draft ? r : r - a.gamma);
  const char* base = static_cast<const char*>(is_draft ? a.draft : a.target);
  return base + idx * a.V * es;
}

// Bounded polls.  A timeout (or an error already recorded by another
// work-group) records the error and returns whatever the word holds.
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
__device__ __forceinline__ uint64_t poll(const VerifyArgs& a, const uint64_t* p) {
  uint64_t w = ld_dev_u64(p);
  unsigned polls = 0;
  while (w == 0ull && !give_up(a, polls)) w = ld_dev_u64(p);
  return w;
}
// The sequence's decision record: thread 0 waits for each word, the
// work-group reads it from LDS (COUNT: thread 0 then counts this item as done
// with the record).  The fields end up in scalar registers.
template <bool COUNT>
__device__ __forceinline__ SeqRec wait_rec(const VerifyArgs& a, int b) {
  __shared__ uint64_t w[kRecWords];
  if (threadIdx.x == 0) {
    // All words are requested together, again until every one has arrived.
    const uint64_t* p = reinterpret_cast<const uint64_t*>(a.seq + b);
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
    for (int i = 0; i < kRecWords; ++i) w[i] = ~v[i];
  }
  __syncthreads();
  SeqRec r;
  uint64_t* rw = reinterpret_cast<uint64_t*>(&r);
#pragma unroll
  for (int i = 0; i < kRecWords; ++i) rw[i] = uni(w[i]);
  if (COUNT) {
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(a.flag + (int64_t)b * kFlagStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return r;
}

// ---------------------------------------------------------------------------
// Stream item: one chunk of one row -> its log2-normaliser piece.

// One batch of N units (8 logits each) of a lane: raise the lane's integer
// offset if the batch holds a larger logit (rescaling the running sum by an
// exact power of two), then add the batch's terms 2^(l c_T - mref), tree-summed
// in fp32, to the fp64 running sum.  LEAD: also track the lane's leader unit
// (units start at jb + u kTile).
template <int DT, bool VEC, int N, bool LEAD = false>
__device__ __forceinline__ void stream_batch(const Raw8<DT, VEC> (&raw)[N], float ch, float cl,
                                             float& mref, float& mraw, double& s, int& pos, int jb) {
  float v[N * 8];
#pragma unroll
  for (int u = 0; u < N; ++u) unpack<DT, VEC>(raw[u], *reinterpret_cast<float(*)[8]>(v + u * 8));
  float um[N];
#pragma unroll
  for (int u = 0; u < N; ++u) {
    um[u] = v[u * 8];
#pragma unroll
    for (int e = 1; e < 8; ++e) um[u] = fmaxf(um[u], v[u * 8 + e]);
  }
  float bm = um[0];
#pragma unroll
  for (int u = 1; u < N; ++u) bm = fmaxf(bm, um[u]);
  if constexpr (LEAD) lead_batch<N>(um, bm, jb, mraw, pos);
  mraw = fmaxf(mraw, bm);
  const float bl = bm * ch;
  if (bl > mref) {
    const float nref = ceilf(fminf(bl, 1.0e30f));
    if (s != 0.0) s = ldexp(s, (int)fmaxf(mref - nref, -2000.f));
    mref = nref;
  }
#pragma unroll
  for (int e = 0; e < N * 8; ++e) v[e] = exp2_fast(fmaf(v[e], cl, fmaf(v[e], ch, -mref)));
#pragma unroll
  for (int w = N * 4; w >= 1; w >>= 1)   // pairwise sum in fp32
#pragma unroll
    for (int e = 0; e < w; ++e) v[e] += v[e + w];
  s += (double)v[0];
}

struct StreamLds {
  float f[2 * kWaves];
  double d[kWaves];
  uint64_t key[kWaves * 3];   // each wave's three best lane leaders
  int nan[kWaves];
};

// The chunk's three best lane leaders (LEAD items): each wave ranks its lanes
// and leaves its three in LDS before the barrier that follows.
__device__ __forceinline__ void wave_leaders(float mx, int pos, StreamLds& sh) {
  uint64_t t[3] = {pos >= 0 ? make_key(__float_as_uint(mx), pos) : 0ull, 0ull, 0ull};
  uint64_t w3[3];
  wave_top3(t, w3);
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int r = 0; r < 3; ++r) sh.key[(threadIdx.x >> 6) * 3 + r] = w3[r];
  }
}
// After that barrier, thread 0: merge the waves' leaders into the record.
__device__ __forceinline__ void store_leaders(const StreamLds& sh, bool nan, Top3* out) {
  uint64_t m[3] = {0, 0, 0};
#pragma unroll
  for (int i = 0; i < kWaves * 3; ++i) insert3(m, sh.key[i]);
  Top3 o;
  o.key[0] = m[0];
  o.key[1] = m[1];
  o.key[2] = m[2];
  o.nan = nan ? 1u : 0u;
  *out = o;
}

// LEAD (draft rows, with outcome prediction): also record the chunk's lane
// leaders in cpart.
template <int DT, bool VEC, int U, bool LEAD = false>
__device__ __forceinline__ void stream_item(const VerifyArgs& a, int b, int r, int c, StreamLds& sh) {
  const void* row = row_ptr<DT>(a, b, r);
  const int64_t begin = (int64_t)c * a.chunk;
  const int64_t end = min<int64_t>(begin + a.chunk, a.V);
  const TCoef tc = temp_coef(a, b);
  const float ch = tc.c_hi, cl = tc.c_lo;

  // mref: this lane's integer offset (log2 units); s: fp64 sum of 2^(l*c_T - mref).
  float mref = kNegSentinel, mraw = -INFINITY;
  double s = 0.0;
  int pos = -1;
  constexpr int64_t kStep = (int64_t)kThreads * kUnit;
  constexpr int64_t kBatch = U * kStep;
  int64_t j;
  if constexpr (VEC) {
    // Full batches (as many in every lane) through a buffer resource over the
    // chunk; the rest of the chunk unit by unit below.
    constexpr int kEs = DT == kBF16 ? 2 : 4;
    const int nb = (int)((end - begin) / kBatch);
    const __amdgpu_buffer_rsrc_t rs =
        chunk_rsrc(static_cast<const char*>(row) + begin * kEs, (int)((end - begin) * kEs));
    const int voff = (int)threadIdx.x * kUnit * kEs;
    for (int i = 0; i < nb; ++i) {
      Raw8<DT, VEC> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        load_raw_buf<DT>(rs, voff, (int)((i * kBatch + u * kStep) * kEs), raw[u]);
      stream_batch<DT, VEC, U, LEAD>(raw, ch, cl, mref, mraw, s, pos,
                                     (int)(begin + i * kBatch) + (int)threadIdx.x * kUnit);
    }
    j = begin + nb * kBatch + (int64_t)threadIdx.x * kUnit;
  } else {
    // Full batches: U units, all in range, loads issued back to back.
    for (j = begin + (int64_t)threadIdx.x * kUnit; j + (U - 1) * kStep + kUnit <= end; j += kBatch) {
      Raw8<DT, VEC> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) load_raw<DT, VEC, true>(row, j + u * kStep, end, raw[u]);
      stream_batch<DT, VEC, U, LEAD>(raw, ch, cl, mref, mraw, s, pos, (int)j);
    }
  }
  // Remaining units of this lane (fewer than U; the last may be partial).
  for (; j < end; j += kStep) {
    Raw8<DT, VEC> raw[1];
    load_raw<DT, VEC, true>(row, j, end, raw[0]);
    stream_batch<DT, VEC, 1, LEAD>(raw, ch, cl, mref, mraw, s, pos, (int)j);
  }
  // Merge the lanes: wave shuffles, then one barrier; thread 0 publishes.
  const float wm = wave_max(mref);
  const float wr = wave_max(mraw);
  double sd = (s != 0.0) ? ldexp(s, (int)fmaxf(mref - wm, -2000.f)) : 0.0;
  sd = wave_sum(sd);
  const int wave = threadIdx.x >> 6;
  if constexpr (LEAD) wave_leaders(mraw, pos, sh);
  if ((threadIdx.x & 63) == 0) {
    sh.f[wave] = wm;
    sh.f[kWaves + wave] = wr;
    sh.d[wave] = sd;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mb = sh.f[0], mr = sh.f[kWaves];
    for (int i = 1; i < kWaves; ++i) {
      mb = fmaxf(mb, sh.f[i]);
      mr = fmaxf(mr, sh.f[kWaves + i]);
    }
    double sb = 0.0;
    for (int i = 0; i < kWaves; ++i)
      if (sh.d[i] != 0.0) sb += ldexp(sh.d[i], (int)fmaxf(sh.f[i] - mb, -2000.f));
    // log2 of the chunk's normaliser; -inf for an all -inf chunk.
    const double v = sb > 0.0 ? (double)mb + log2(sb) : (sb == 0.0 ? -INFINITY : sb);
    const int64_t idx = ((int64_t)b * (2 * a.gamma + 1) + r) * a.nc + c;
    slot_put32(a.mraw + idx, mr);
    slot_put(a.part + idx, v);
    if constexpr (LEAD) store_leaders(sh, v != v, a.cpart + ((int64_t)b * (a.gamma + 1) + r) * a.nc + c);
  }
}

// Draft row gamma (outcome prediction only): one chunk's lane leaders and
// NaN flag, nothing else.
template <int DT, bool VEC, int U>
__device__ void leader_item(const VerifyArgs& a, int b, int c, StreamLds& sh) {
  constexpr int kEs = DT == kBF16 ? 2 : 4;
  const int64_t ridx = (int64_t)b * (a.gamma + 1) + a.gamma;
  const void* row = static_cast<const char*>(a.draft) + ridx * a.V * kEs;
  const int64_t begin = (int64_t)c * a.chunk;
  const int64_t end = min<int64_t>(begin + a.chunk, a.V);
  float mx = -INFINITY;
  int pos = -1;
  bool nan = false;
  constexpr int64_t kStep = (int64_t)kThreads * kUnit;
  constexpr int64_t kBatch = U * kStep;
  auto batch = [&](const auto& raw, auto n, int jb) {
    constexpr int N = decltype(n)::value;
    float um[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
      float v[8];
      unpack<DT, VEC>(raw[u], v);
      um[u] = v[0];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        nan = nan || v[e] != v[e];
        um[u] = fmaxf(um[u], v[e]);
      }
    }
    float bm = um[0];
#pragma unroll
    for (int u = 1; u < N; ++u) bm = fmaxf(bm, um[u]);
    lead_batch<N>(um, bm, jb, mx, pos);
    mx = fmaxf(mx, bm);
  };
  int64_t j;
  if constexpr (VEC) {
    const int nb = (int)((end - begin) / kBatch);
    const __amdgpu_buffer_rsrc_t rs =
        chunk_rsrc(static_cast<const char*>(row) + begin * kEs, (int)((end - begin) * kEs));
    const int voff = (int)threadIdx.x * kUnit * kEs;
    for (int i = 0; i < nb; ++i) {
      Raw8<DT, VEC> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        load_raw_buf<DT>(rs, voff, (int)((i * kBatch + u * kStep) * kEs), raw[u]);
      batch(raw, std::integral_constant<int, U>{}, (int)(begin + i * kBatch) + (int)threadIdx.x * kUnit);
    }
    j = begin + nb * kBatch + (int64_t)threadIdx.x * kUnit;
  } else {
    j = begin + (int64_t)threadIdx.x * kUnit;
  }
  for (; j < end; j += kStep) {
    Raw8<DT, VEC> raw[1];
    load_raw<DT, VEC, true>(row, j, end, raw[0]);
    batch(raw, std::integral_constant<int, 1>{}, (int)j);
  }
  wave_leaders(mx, pos, sh);
  const bool wn = __ballot(nan) != 0;
  if ((threadIdx.x & 63) == 0) sh.nan[threadIdx.x >> 6] = wn ? 1 : 0;
  __syncthreads();
  if (threadIdx.x == 0) {
    int any = 0;
    for (int i = 0; i < kWaves; ++i) any |= sh.nan[i];
    store_leaders(sh, any != 0, a.cpart + ridx * a.nc + c);
  }
}

// The outputs of an invalid sequence (threads 0..gamma).
__device__ __forceinline__ void write_invalid(const VerifyArgs& a, int b, int tid) {
  const int g = a.gamma;
  if (tid <= g) a.out_tokens[(int64_t)b * (g + 1) + tid] = -1;
  if (tid == 0) {
    a.out_acc[b] = -1;
    if (a.out_first_reject) a.out_first_reject[b] = -1;
    if (a.out_mask) a.out_mask[b] = 0;
    if (a.out_len) a.out_len[b] = a.in_len ? a.in_len[b] : 0;
  }
}

// ---------------------------------------------------------------------------
// Decision of one sequence.

// Merge the chunk pieces of row r of sequence b within a 16-lane group (lane
// `sub` takes pieces sub, sub + 16, ...): M = the integer ceiling of
// max_c v_c, z = sum_c 2^(v_c - M) (fp64), mr = the row's largest raw logit.
// Waits for every piece (both words of a piece together) and clears them once
// read.  Every lane of the group returns the row's values.
__device__ void merge_row(const VerifyArgs& a, int b, int r, int sub, double& M, double& z, float& mr) {
  const int64_t p0 = ((int64_t)b * (2 * a.gamma + 1) + r) * a.nc;
  M = -INFINITY;
  z = 0.0;
  mr = -INFINITY;
  double v0 = -INFINITY;   // the first piece stays in a register, later ones are read again
  for (int c = sub; c < a.nc; c += 16) {
    uint64_t wv = ld_dev_u64(a.part + p0 + c);
    unsigned wm = __hip_atomic_load(a.mraw + p0 + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned polls = 0;
    while ((wv == 0ull || wm == 0u) && !give_up(a, polls)) {
      if (wv == 0ull) wv = ld_dev_u64(a.part + p0 + c);
      if (wm == 0u) wm = __hip_atomic_load(a.mraw + p0 + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const double v = slot_value(wv);
    mr = fmaxf(mr, __uint_as_float(~wm));
    if (c == sub) v0 = v;
    M = fmax(M, v);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
    M = fmax(M, __shfl_xor(M, o, 16));
    mr = fmaxf(mr, __shfl_xor(mr, o, 16));
  }
  M = ceil(M);
  for (int c = sub; c < a.nc; c += 16) {
    const double v = c == sub ? v0 : slot_value(ld_dev_u64(a.part + p0 + c));
    if (v != -INFINITY) z += exp2(v - M);   // a NaN piece stays NaN
    slot_clear(a.part + p0 + c);
    slot_clear32(a.mraw + p0 + c);
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) z += __shfl_xor(z, o, 16);
}

// An all -inf row (M = -inf), a +inf logit (M = +inf) or a NaN logit (z =
// NaN) makes a row bad.
__device__ __forceinline__ bool row_ok(double M, double z) {
  return (z > 0.0) && isfinite(z) && isfinite(M);
}

struct DecideLds {
  double M[128];   // row offsets (integers, log2 units)
  double Z[128];   // row normalisers: sum_j 2^(l_j c_T - M)
  float mr[128];   // row maxima of the raw logits
  int bad[128];
  int x[64];       // draft tokens, their draft and target logits, accept uniforms
  float ldx[64], ltx[64], ux[64];
  uint64_t mask;
  int k, valid;
};

// The rows the accept tests read, draft rows 0..gamma-1 and target rows
// 0..gamma-1 (16 lanes per row, 12 rows per pass), then the accept test at
// every draft position (wave 0, lane i = position i; fp64) and the decision
// record.  Target row gamma is checked by the sequence's final item.  A bad
// row or token makes the sequence invalid here, with its outputs.
template <int DT, bool CUT = false>
__device__ void decide_item(const VerifyArgs& a, int b, DecideLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = a.gamma, Rd = 2 * g, R = 2 * g + 1;
  // Wave 1 gathers the draft tokens' logits and the uniforms (independent of
  // the row pieces) while waves 0, 2 and 3 merge the pieces.
  if (wave == 1) {
    if (lane < g) {
      const int x = a.tokens[(int64_t)b * g + lane];
      float ldx = 0.f, ltx = 0.f;
      if (x >= 0 && x < a.V) {
        ldx = load_one<DT>(row_ptr<DT>(a, b, lane), x);
        ltx = load_one<DT>(row_ptr<DT>(a, b, g + lane), x);
      }
      sh.x[lane] = x;
      sh.ldx[lane] = ldx;
      sh.ltx[lane] = ltx;
      sh.ux[lane] = a.u_acc[(int64_t)b * g + lane];
    }
  } else {
    for (int r0 = 0; r0 < Rd; r0 += 12) {
      const int r = r0 + (wave == 0 ? 0 : wave - 1) * 4 + (lane >> 4);
      if (r < Rd) {
        double M, z;
        float mr;
        merge_row(a, b, r, lane & 15, M, z, mr);
        if ((lane & 15) == 0) {
          sh.M[r] = M;
          sh.Z[r] = z;
          sh.mr[r] = mr;
          sh.bad[r] = !row_ok(M, z);
        }
      }
    }
  }
  __syncthreads();
  const TCoef tc = temp_coef(a, b);
  for (int r = tid; r < Rd; r += kThreads) {
    if (sh.bad[r]) continue;
    if (a.diag.row_max) a.diag.row_max[(int64_t)b * R + r] = (double)sh.mr[r] * tc.invT;
    if (a.diag.row_logZ) a.diag.row_logZ[(int64_t)b * R + r] = sh.M[r] * 0.69314718055994530942 + log(sh.Z[r]);
  }

  if (wave == 0) {
    int rows_bad = 0;
    for (int r = lane; r < Rd; r += 64) rows_bad |= sh.bad[r];
    rows_bad = __ballot(rows_bad) != 0 || (a.temps && !temp_ok(seq_temp(a, b)));
    int acc = 0, bad = 0;
    if (lane < g) {
      const int x = sh.x[lane];
      bad = (x < 0 || x >= a.V);
      if (!bad && !rows_bad) {
        // p(x) = pn / Zd and q(x) = qn / Zt; the ratio with one division.
        double pn = exp2((double)sh.ldx[lane] * tc.cTd - sh.M[lane]);
        double qn = exp2((double)sh.ltx[lane] * tc.cTd - sh.M[g + lane]);
        if constexpr (CUT) {   // p'(x) = p(x) / P_d inside the draft nucleus, else 0; q' alike
          const TopPRow* tp = a.topp + (int64_t)b * R;
          pn = sh.ldx[lane] >= tp[lane].L ? pn / tp[lane].P : 0.0;
          qn = sh.ltx[lane] >= tp[g + lane].L ? qn / tp[g + lane].P : 0.0;
        }
        double ratio;
        if (pn > 0.0) ratio = fmin(1.0, (qn * sh.Z[lane]) / (pn * sh.Z[g + lane]));
        else ratio = qn > 0.0 ? 1.0 : 0.0;
        acc = (double)sh.ux[lane] < ratio;
        if (a.diag.px) a.diag.px[(int64_t)b * g + lane] = pn / sh.Z[lane];
        if (a.diag.qx) a.diag.qx[(int64_t)b * g + lane] = qn / sh.Z[g + lane];
      }
    }
    const uint64_t mask = __ballot(acc);
    const uint64_t badm = __ballot(bad);
    if (lane == 0) {
      sh.mask = mask & ((1ull << g) - 1);
      sh.valid = !rows_bad && badm == 0;
      sh.k = min(g, __ffsll((unsigned long long)~mask) - 1);
    }
  }
  __syncthreads();

  const int k = sh.k;
  if (!sh.valid) write_invalid(a, b, tid);
  if (tid == 0) {
    SeqRec rec;
    rec.mask = sh.mask;
    rec.k = k;
    rec.valid = sh.valid;
    rec.mode = k == g ? kModeTarget
                      : (!a.saguaro ? kModeResidual : (a.eps > 0.f ? kModeSaguaroEps : kModeSaguaro));
    rec.Mt = 0.f;
    rec.K_hi = rec.K_lo = 0.f;
    rec.Zt = 1.0;
    if (sh.valid && k < g) {   // the bonus draw (k == gamma) offsets each tile on its own
      const double Mt = sh.M[g + k];
      double Pt = 1.0, Pd = 1.0;   // nucleus masses (top-p): q' = q / Pt, p' = p / Pd
      if constexpr (CUT) {
        Pt = a.topp[(int64_t)b * R + g + k].P;
        Pd = a.topp[(int64_t)b * R + k].P;
      }
      rec.Mt = (float)Mt;   // exact below 2^24; otherwise Zt absorbs the rounding
      rec.Zt = ldexp(sh.Z[g + k] * Pt, (int)fmin(fmax(Mt - (double)rec.Mt, -2000.0), 2000.0));
      const double K = (Mt - sh.M[k]) + log2((sh.Z[g + k] * Pt) / (sh.Z[k] * Pd));
      rec.K_hi = (float)K;
      rec.K_lo = (float)(K - (double)rec.K_hi);
    }
    store_rec(a.seq + b, rec);
  }
}

// ---------------------------------------------------------------------------
// Early exit: the accept test of one position ("Speculative Decoding: small
// model guesses, large model verifies", section 3: test position i only once
// every earlier position was accepted; stop at the first rejection).

struct TestLds {
  double M[2], Z[2];
  float mr[2];
  int bad[2];
  int x;
  float ldx, ltx, ux;
  int decided, acc, bad_all;
};

// Position i of sequence b: merges (and clears) the pieces of draft row i and
// target row i, tests the position, and publishes a rejection (or a bad row
// or token) at once through the stop word, so later positions' stream items
// skip their rows.  It then waits for the earlier positions - every one
// accepted (the progress word reaches i) or one of them stopped the sequence
// - which are decided by items with smaller block numbers.  If every earlier
// position was accepted, this item decides: it advances the progress word
// (accepted, more positions follow) or writes the decision record (rejected,
// invalid, or the last position accepted).
template <int DT>
__device__ void test_item(const VerifyArgs& a, int b, int i, TestLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = a.gamma, R = 2 * g + 1;
  unsigned* fl = a.flag + (int64_t)b * kFlagStride;
  if (wave == 0) {
    if (lane < 32) {
      const int h = lane >> 4;   // 0: draft row i, 1: target row i
      double M, z;
      float mr;
      merge_row(a, b, h ? g + i : i, lane & 15, M, z, mr);
      if ((lane & 15) == 0) {
        sh.M[h] = M;
        sh.Z[h] = z;
        sh.mr[h] = mr;
        sh.bad[h] = !row_ok(M, z);
      }
    }
  } else if (wave == 1 && lane == 0) {
    const int x = a.tokens[(int64_t)b * g + i];
    float ldx = 0.f, ltx = 0.f;
    if (x >= 0 && x < a.V) {
      ldx = load_one<DT>(row_ptr<DT>(a, b, i), x);
      ltx = load_one<DT>(row_ptr<DT>(a, b, g + i), x);
    }
    sh.x = x;
    sh.ldx = ldx;
    sh.ltx = ltx;
    sh.ux = a.u_acc[(int64_t)b * g + i];
  }
  __syncthreads();
  if (tid == 0) {
    const TCoef tc = temp_coef(a, b);
    const int x = sh.x;
    const bool bad = x < 0 || x >= a.V || sh.bad[0] || sh.bad[1] || (a.temps && !temp_ok(seq_temp(a, b)));
    bool acc = false;
    double pn = 0.0, qn = 0.0;
    if (!bad) {
      pn = exp2((double)sh.ldx * tc.cTd - sh.M[0]);
      qn = exp2((double)sh.ltx * tc.cTd - sh.M[1]);
      double ratio;
      if (pn > 0.0) ratio = fmin(1.0, (qn * sh.Z[0]) / (pn * sh.Z[1]));
      else ratio = qn > 0.0 ? 1.0 : 0.0;
      acc = (double)sh.ux < ratio;
    }
    const unsigned mine = 64u - (unsigned)i;
    if (bad || !acc) __hip_atomic_fetch_max(fl + kStopWord, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool decided = false;
    if (i == 0) {
      decided = true;
    } else {
      unsigned polls = 0;
      for (;;) {
        if (ld_dev_u32(fl + kStopWord) > mine) break;              // an earlier position stopped it
        if (ld_dev_u32(fl + kProgWord) >= (unsigned)i) {           // every earlier one accepted
          decided = true;
          break;
        }
        if (give_up(a, polls)) break;
      }
    }
    if (decided && !bad && acc && i + 1 < g)
      __hip_atomic_store(fl + kProgWord, (unsigned)(i + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (decided && !bad) {
      if (a.diag.px) a.diag.px[(int64_t)b * g + i] = pn / sh.Z[0];
      if (a.diag.qx) a.diag.qx[(int64_t)b * g + i] = qn / sh.Z[1];
      if (a.diag.row_max) {
        a.diag.row_max[(int64_t)b * R + i] = (double)sh.mr[0] * tc.invT;
        a.diag.row_max[(int64_t)b * R + g + i] = (double)sh.mr[1] * tc.invT;
      }
      if (a.diag.row_logZ) {
        a.diag.row_logZ[(int64_t)b * R + i] = sh.M[0] * 0.69314718055994530942 + log(sh.Z[0]);
        a.diag.row_logZ[(int64_t)b * R + g + i] = sh.M[1] * 0.69314718055994530942 + log(sh.Z[1]);
      }
    }
    sh.decided = decided && (bad || !acc || i + 1 == g);
    sh.acc = acc;
    sh.bad_all = bad;
    __hip_atomic_fetch_add(fl + kTestsWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!sh.decided) return;
  const bool valid = !sh.bad_all;
  const int k = valid && sh.acc ? g : i;
  if (!valid) write_invalid(a, b, tid);
  if (tid == 0) {
    SeqRec rec;
    rec.mask = (k >= 64) ? ~0ull : ((1ull << k) - 1);
    rec.k = k;
    rec.valid = valid;
    rec.mode = k == g ? kModeTarget
                      : (!a.saguaro ? kModeResidual : (a.eps > 0.f ? kModeSaguaroEps : kModeSaguaro));
    rec.Mt = 0.f;
    rec.K_hi = rec.K_lo = 0.f;
    rec.Zt = 1.0;
    if (valid && k < g) {
      const double Mt = sh.M[1];
      rec.Mt = (float)Mt;
      rec.Zt = ldexp(sh.Z[1], (int)fmin(fmax(Mt - (double)rec.Mt, -2000.0), 2000.0));
      const double K = (Mt - sh.M[0]) + log2(sh.Z[1] / sh.Z[0]);
      rec.K_hi = (float)K;
      rec.K_lo = (float)(K - (double)rec.K_hi);
    }
    store_rec(a.seq + b, rec);
  }
}

// ---------------------------------------------------------------------------
// Sampling weights.

struct SampleCoef {
  float c_hi, c_lo, Mt, K_hi, K_lo, epsS;
  float A_hi, A_lo;   // K - Mt as an unevaluated float pair: p_j ~ 2^(ld_j c_T + K - Mt)
  float Ld, Lt;       // top-p thresholds of the rows drawn from (-inf: no cut)
};

// A top-p cut: logits below the row's threshold act as -inf (probability 0);
// the renormalisation is folded into the decision record's constants.
template <bool CUT>
__device__ __forceinline__ void cut8(float (&v)[8], float L) {
  if constexpr (CUT) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] >= L ? v[e] : -INFINITY;
  }
}
template <bool CUT>
__device__ __forceinline__ float cut1(float v, float L) {
  if constexpr (CUT) return v >= L ? v : -INFINITY;
  else return v;
}

template <bool CUT = false>
__device__ __forceinline__ SampleCoef coef_of(const VerifyArgs& a, int b, const SeqRec& rec, float epsS) {
  SampleCoef c;
  const TCoef tc = temp_coef(a, b);
  c.c_hi = tc.c_hi;
  c.c_lo = tc.c_lo;
  c.Mt = rec.Mt;
  c.K_hi = rec.K_hi;
  c.K_lo = rec.K_lo;
  c.epsS = epsS;
  const double A = ((double)rec.K_hi + (double)rec.K_lo) - (double)rec.Mt;
  c.A_hi = uni((float)A);
  c.A_lo = uni((float)(A - (double)c.A_hi));
  c.Ld = -INFINITY;
  c.Lt = -INFINITY;
  if (CUT && a.topp && rec.k >= 0 && rec.k <= a.gamma) {
    const TopPRow* tp = a.topp + (int64_t)b * (2 * a.gamma + 1);
    c.Lt = uni(tp[a.gamma + rec.k].L);
    if (rec.k < a.gamma) c.Ld = uni(tp[rec.k].L);
  }
  return c;
}

constexpr float kLn2f = 0.69314718055994530942f;

// 1 - 2^d.  PRECISE: for d in (-1, 0], -expm1(d ln 2) by its Taylor series
// (degree 9, truncation below 1e-8 relative), so a small residual keeps its
// relative precision; otherwise (and for d <= -1) 1 - 2^d from the rounded
// exponential, whose error is a few ulp of 1 (of q_j, not of the residual).
template <bool PRECISE>
__device__ __forceinline__ float one_minus_exp2(float d, float ex) {
  if constexpr (!PRECISE) {
    return 1.f - ex;
  } else {
    const float x = d * kLn2f;
    float p = 1.f / 362880.f;
    p = fmaf(p, x, 1.f / 40320.f);
    p = fmaf(p, x, 1.f / 5040.f);
    p = fmaf(p, x, 1.f / 720.f);
    p = fmaf(p, x, 1.f / 120.f);
    p = fmaf(p, x, 1.f / 24.f);
    p = fmaf(p, x, 1.f / 6.f);
    p = fmaf(p, x, 0.5f);
    p = fmaf(p, x, 1.f);
    return d > -1.f ? -x * p : 1.f - ex;
  }
}

// Sampling weight of one logit pair, proportional (one factor per sequence)
// to the probability of the distribution drawn from:
//   target row:  q_j                      (eq_j = 2^(lt_j c_T - Mt))
//   residual:    (q_j - p_j)+             (eq_j (1 - 2^delta_j) where delta_j < 0)
//   Saguaro:     sqrt(p_j (q_j - p_j)+)   (eq_j sqrt(2^delta_j (1 - 2^delta_j)))
//   Saguaro eps: sqrt(p_j max(r_j, eps))  (sqrt(eq_j 2^delta_j max(res_j, eps sum res)))
// with delta_j = log2(p_j / q_j) = (ld_j - lt_j) c_T + K (exact logit
// difference for bf16, a two-sum for float32).  r = the residual weight.
template <int DT, int MODE, bool PRECISE>
__device__ __forceinline__ float weight_one(float ld, float lt, const SampleCoef& c, float& r) {
  const float eq = exp2_fast(fmaf(lt, c.c_lo, fmaf(lt, c.c_hi, -c.Mt)));
  if constexpr (MODE == kModeTarget) {
    r = 0.f;
    return eq;
  } else if constexpr (MODE == kModeResidual && !PRECISE) {
    // (q_j - p_j)+ from both scaled probabilities: the same absolute error
    // (a few ulp of q_j) as 1 - 2^delta_j, with fewer instructions.
    const float ep = exp2_fast(fmaf(ld, c.c_lo, fmaf(ld, c.c_hi, c.A_hi) + c.A_lo));
    const float res = fmaxf(eq - ep, 0.f);
    r = res;
    return res;
  } else {
    const float dl = ld - lt;
    float d;
    if constexpr (DT == kBF16) {
      d = fmaf(dl, c.c_hi, c.K_hi) + fmaf(dl, c.c_lo, c.K_lo);   // dl is exact
    } else {
      const float bb = dl - ld;
      const float err = (ld - (dl - bb)) - (lt + bb);             // ld - lt = dl + err
      d = fmaf(dl, c.c_hi, c.K_hi) + fmaf(err, c.c_hi, fmaf(dl, c.c_lo, c.K_lo));
      if (ld == -INFINITY) d = -INFINITY;   // p_j = 0 (the two-sum of an infinite difference is NaN)
    }
    const float ex = exp2_fast(d);          // p_j / q_j
    const float em1 = one_minus_exp2<PRECISE>(d, ex);
    const bool pos = (eq > 0.f) && (d < 0.f);
    const float res = pos ? eq * em1 : 0.f;
    r = res;
    if constexpr (MODE == kModeResidual) return res;
    else if constexpr (MODE == kModeSaguaro) return pos ? eq * sqrtf(ex * em1) : 0.f;
    else {   // p_j from its own exponential where q_j = 0 (eq ex would be 0 * inf)
      const float pj = eq > 0.f ? eq * ex : exp2_fast(fmaf(ld, c.c_lo, fmaf(ld, c.c_hi, c.A_hi) + c.A_lo));
      return sqrtf(pj * fmaxf(res, c.epsS));
    }
  }
}

template <int DT, int MODE, bool PRECISE>
__device__ __forceinline__ void sample_weights(const float (&ld)[8], const float (&lt)[8],
                                               const SampleCoef& c, float (&w)[8], float (&r)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = weight_one<DT, MODE, PRECISE>(ld[e], lt[e], c, r[e]);
}

// Call f with the weight mode as a compile-time constant.  EPS = false: code
// that never sees the Saguaro eps > 0 mode (the fused kernel) leaves it out.
template <bool EPS = true, class F>
__device__ __forceinline__ void with_mode(int mode, F&& f) {
  switch (mode) {
    case kModeTarget: f(std::integral_constant<int, kModeTarget>{}); break;
    case kModeResidual: f(std::integral_constant<int, kModeResidual>{}); break;
    case kModeSaguaro: f(std::integral_constant<int, kModeSaguaro>{}); break;
    default:
      if constexpr (EPS) f(std::integral_constant<int, kModeSaguaroEps>{});
      break;
  }
}

// Rows of the draw: target row k and (on a rejection) draft row k.
template <int DT>
__device__ __forceinline__ void draw_rows(const VerifyArgs& a, int b, int k, const void*& drow,
                                          const void*& trow) {
  drow = row_ptr<DT>(a, b, k < a.gamma ? k : 0);
  trow = row_ptr<DT>(a, b, a.gamma + k);
}

// Integer offset of a tile of target logits for the bonus draw (log2 units):
// the ceiling of its largest logit times c_T; 0 for an all -inf tile.
__device__ __forceinline__ float tile_offset(float bm, float c_hi) {
  const float bl = bm * c_hi;
  return bl > -1.0e30f ? ceilf(fminf(bl, 1.0e30f)) : 0.f;
}

// Tile sums of the weights over tiles [t0, t0 + N) (clipped to ntile): tw[i]
// (fp64, identical in every thread) and, last, the residual total.  The loads
// of G tiles are in flight together (all N for packed bf16 rows, whose raw
// words take half the registers of floats).  In target mode (the bonus draw)
// every tile gets its own integer offset mt[i] (its weights are
// 2^(lt_j c_T - mt[i])), so no row normaliser is needed.
template <int DT, bool VEC, int MODE, bool CUT = false, int N = kTilesPerItem>
__device__ __forceinline__ void tile_sums(const VerifyArgs& a, int b, const SampleCoef& cf, int k,
                                          int t0, double (&tw)[N + 1], float (&mt)[N], double* lds_d) {
  constexpr int G = (DT == kBF16 && VEC) ? N : (N >= 2 ? 2 : 1);
  static_assert(N % G == 0, "tile groups must divide the item");
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  const int64_t lane_off = (int64_t)threadIdx.x * kUnit;
  float rs = 0.f;
#pragma unroll
  for (int g0 = 0; g0 < N; g0 += G) {
    Raw8<DT, VEC> rd[G], rt[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int t = t0 + g0 + i;
      const int64_t j0 = t < a.ntile ? (int64_t)t * kTile + lane_off : (int64_t)a.V;
      load_raw<DT, VEC, kSampleNT>(trow, j0, a.V, rt[i]);
      if constexpr (MODE != kModeTarget) load_raw<DT, VEC, kSampleNT>(drow, j0, a.V, rd[i]);
    }
    float off[G];
    if constexpr (MODE == kModeTarget) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        float lt[8];
        unpack<DT, VEC>(rt[i], lt);
        cut8<CUT>(lt, cf.Lt);
        float m = lt[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) m = fmaxf(m, lt[e]);
        off[i] = m;
      }
      block_max_n<G>(off, reinterpret_cast<float*>(lds_d));
#pragma unroll
      for (int i = 0; i < G; ++i) off[i] = tile_offset(off[i], cf.c_hi);
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      float ld[8], lt[8], w[8], r[8];
      unpack<DT, VEC>(rt[i], lt);
      cut8<CUT>(lt, cf.Lt);
      if constexpr (MODE != kModeTarget) {
        unpack<DT, VEC>(rd[i], ld);
        cut8<CUT>(ld, cf.Ld);
      }
      SampleCoef c = cf;
      if constexpr (MODE == kModeTarget) {
        c.Mt = off[i];
        mt[g0 + i] = off[i];
      }
      sample_weights<DT, MODE, false>(ld, lt, c, w, r);
      float ws = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ws += w[e];
        if constexpr (MODE == kModeSaguaro || MODE == kModeSaguaroEps) rs += r[e];
      }
      if constexpr (MODE == kModeResidual) rs += ws;   // the residual-mass items read it
      tw[g0 + i] = (double)ws;
    }
    if constexpr (G < N) __builtin_amdgcn_sched_barrier(0);   // keep the groups apart
  }
  tw[N] = (double)rs;
  block_sum_n<N + 1>(tw, lds_d);
}

// A tile's slot value: the plain sum, or in target mode log2 of it with the
// tile's offset added (-inf for an empty tile).
__device__ __forceinline__ double tile_slot_value(int mode, double sum, float off) {
  if (mode != kModeTarget) return sum;
  return sum > 0.0 ? (double)off + log2(sum) : (sum == 0.0 ? -INFINITY : sum);
}

// eps * (residual mass) for Saguaro eps > 0, from the residual-mass items'
// slots (waited for), summed in the same order by every reader.
__device__ float eps_clamp(const VerifyArgs& a, int b, double* lds_d) {
  double v = 0.0;
  for (int i = threadIdx.x; i < a.nt; i += kThreads) v += slot_value(poll(a, a.mass + (int64_t)b * a.nt + i));
  v = block_sum(v, lds_d);
  return uni((float)(v * (double)a.eps));
}

// ---------------------------------------------------------------------------
// Residual-mass and sampling items.

template <int DT, bool VEC, bool CUT = false>
__device__ void mass_item(const VerifyArgs& a, int b, int s, double* lds_d) {
  const SeqRec rec = wait_rec<true>(a, b);
  if (!rec.valid || rec.mode != kModeSaguaroEps) return;
  double tw[kTilesPerItem + 1];
  float mt[kTilesPerItem];
  tile_sums<DT, VEC, kModeResidual, CUT>(a, b, coef_of<CUT>(a, b, rec, 0.f), rec.k, s * kTilesPerItem, tw, mt, lds_d);
  if (threadIdx.x == 0) slot_put(a.mass + (int64_t)b * a.nt + s, tw[kTilesPerItem]);
}

template <int DT, bool VEC, bool CUT = false, bool EPS = true>
__device__ void sample_item(const VerifyArgs& a, int b, int s, double* lds_d) {
  const SeqRec rec = wait_rec<true>(a, b);
  if (!rec.valid) return;
  const int t0 = s * kTilesPerItem;
  const float epsS = rec.mode == kModeSaguaroEps ? eps_clamp(a, b, lds_d) : 0.f;
  const SampleCoef cf = coef_of<CUT>(a, b, rec, epsS);
  with_mode<EPS>(rec.mode, [&](auto m) {
    constexpr int MODE = decltype(m)::value;
    double tw[kTilesPerItem + 1];
    float mt[kTilesPerItem];
    tile_sums<DT, VEC, MODE, CUT>(a, b, cf, rec.k, t0, tw, mt, lds_d);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int i = 0; i < kTilesPerItem; ++i)
        if (t0 + i < a.ntile)
          slot_put(a.tiles + (int64_t)b * a.ntile + t0 + i, tile_slot_value(MODE, tw[i], mt[i]));
      if (MODE == kModeSaguaro) slot_put(a.rsum + (int64_t)b * a.nt + s, tw[kTilesPerItem]);
    }
  });
}

// ---------------------------------------------------------------------------
// Draw item.

struct DrawLds {
  double lds_d[kWaves * (kTilesPerItem + 1)];
  int lds_i[kWaves];
  int tile, y, e;   // chosen tile, drawn token, tile units = 2^e draw units
  double off, lane_off, lo, hi, Mp;
  float w8[kUnit];
};

__device__ __forceinline__ double tile_value(const uint64_t* tiles, int t) {
  return slot_value(ld_dev_u64(tiles + t));
}

// Target-mode tile values hold v_t = offset + log2(sum): replace each by the
// sum in draw units, 2^(v_t - Mp) with Mp the integer ceiling of the largest
// v_t, in place (the slots belong to the draw now).  Sets sh.Mp.
__device__ void tiles_to_linear(uint64_t* tiles, int ntile, DrawLds& sh) {
  const int tid = threadIdx.x;
  float m = -INFINITY;   // an upper bound to within float rounding is all Mp needs
  for (int t = tid; t < ntile; t += kThreads) m = fmaxf(m, (float)tile_value(tiles, t));
  m = block_max(m, reinterpret_cast<float*>(sh.lds_d));
  const double Mp = isfinite(m) ? ceil((double)m) + 1.0 : 0.0;
  for (int t = tid; t < ntile; t += kThreads) {
    const double v = tile_value(tiles, t);
    slot_put(tiles + t, v > -INFINITY ? exp2(v - Mp) : 0.0);
  }
  if (tid == 0) sh.Mp = Mp;
  wait_mem();
  __syncthreads();
}

// Locate the tile holding u * S (S = sum of the tile values) by an fp64 scan
// over the tile values in token order; returns S, sets sh.tile and sh.off.
__device__ double locate_tile(const uint64_t* tiles, int ntile, double u, DrawLds& sh, double& target) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.tile = -1;
  double S = 0.0;
  if (ntile <= kThreads) {   // one tile value per thread, loaded once
    const double v = tid < ntile ? tile_value(tiles, tid) : 0.0;
    double tot;
    const double off = block_exclusive_scan(v, sh.lds_d, tot);
    S = tot;
    target = u * S;
    const int hit = (tid < ntile && off <= target && target < off + v) ? tid : INT_MAX;
    const int first = block_min_int(hit, sh.lds_i);
    if (first != INT_MAX && tid == first) {
      sh.tile = tid;
      sh.off = off;
    }
  } else {
    double v = 0.0;
    for (int i = tid; i < ntile; i += kThreads) v += tile_value(tiles, i);
    S = block_sum(v, sh.lds_d);
    target = u * S;
    double carry = 0.0;
    for (int base = 0; base < ntile; base += kThreads) {
      const int t = base + tid;
      const double x = t < ntile ? tile_value(tiles, t) : 0.0;
      double tot;
      const double off = carry + block_exclusive_scan(x, sh.lds_d, tot);
      const int hit = (t < ntile && off <= target && target < off + x) ? t : INT_MAX;
      const int first = block_min_int(hit, sh.lds_i);
      if (first != INT_MAX) {
        if (t == first) {
          sh.tile = t;
          sh.off = off;
        }
        break;
      }
      carry += tot;
    }
  }
  __syncthreads();
  if (sh.tile < 0) {   // u * S at or past the last running sum (rounding): last nonzero tile
    int last = -1;
    for (int t = tid; t < ntile; t += kThreads)
      if (tile_value(tiles, t) > 0.0) last = t;
    last = -block_min_int(-last, sh.lds_i);
    if (tid == 0) {
      sh.tile = max(last, 0);
      double off = 0.0;
      for (int t = 0; t < last; ++t) off += tile_value(tiles, t);
      sh.off = off;
    }
    __syncthreads();
  }
  return S;
}

// Rescan the chosen tile: the same weights and per-lane fp32 sums as its tile
// sum, fp64 prefix over the lanes, in tile units (one tile unit is 2^e draw
// units; e = 0 but for the bonus draw, where it is the tile's offset minus Mp).
// The lane holding the target (else the last lane with weight) hands its
// eight weights to thread 0, which walks them in fp64: y = the first token
// with weight whose running sum passes the target (else the lane's last token
// with weight).  Sets sh.y, sh.e, sh.lo = C_{y-1} and sh.hi = C_y (draw units).
template <int DT, bool VEC, int MODE, bool CUT = false>
__device__ void rescan_tile(const VerifyArgs& a, int b, int k, const SampleCoef& cf, double target,
                            DrawLds& sh) {
  const int tid = threadIdx.x;
  const int tsel = sh.tile;
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  const int64_t j0 = (int64_t)tsel * kTile + (int64_t)tid * kUnit;
  float w[8];
  int e = 0;
  {
    Raw8<DT, VEC> rd, rt;
    load_raw<DT, VEC>(trow, j0, a.V, rt);
    if constexpr (MODE != kModeTarget) load_raw<DT, VEC>(drow, j0, a.V, rd);
    float ld[8], lt[8], r[8];
    unpack<DT, VEC>(rt, lt);
    cut8<CUT>(lt, cf.Lt);
    if constexpr (MODE != kModeTarget) {
      unpack<DT, VEC>(rd, ld);
      cut8<CUT>(ld, cf.Ld);
    }
    SampleCoef c = cf;
    if (MODE == kModeTarget && k == a.gamma) {   // the bonus draw: the tile's own offset
      float m[1] = {lt[0]};
#pragma unroll
      for (int i = 1; i < 8; ++i) m[0] = fmaxf(m[0], lt[i]);
      block_max_n<1>(m, reinterpret_cast<float*>(sh.lds_d));
      c.Mt = tile_offset(m[0], cf.c_hi);
      e = (int)fmin(fmax((double)c.Mt - sh.Mp, -2000.0), 2000.0);
    }
    sample_weights<DT, MODE, false>(ld, lt, c, w, r);
  }
  float ws = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ws += w[i];
  double tile_tot;
  const double off = block_exclusive_scan((double)ws, sh.lds_d, tile_tot);
  const double tgt = ldexp(target - sh.off, -e);   // in tile units
  const int hit = (ws > 0.f && off <= tgt && tgt < off + (double)ws) ? tid : INT_MAX;
  int owner = block_min_int(hit, sh.lds_i);
  if (owner == INT_MAX) owner = -block_min_int(ws > 0.f ? -tid : 1, sh.lds_i);   // last lane with weight
  if (tid == owner) {
#pragma unroll
    for (int i = 0; i < 8; ++i) sh.w8[i] = w[i];
    sh.lane_off = off;
  }
  __syncthreads();
  if (tid == 0) {
    sh.e = e;
    if (owner < 0) {   // no weight in the tile (not reached: its tile value was positive)
      sh.y = (int)min<int64_t>(a.V - 1, (int64_t)tsel * kTile + kTile - 1);
      sh.lo = sh.hi = sh.off + ldexp(tile_tot, e);
    } else {
      double run = sh.lane_off;
      int idx = -1, last = -1;
      double lo_last = run, lo = run;
      for (int i = 0; i < 8; ++i) {
        const double we = (double)sh.w8[i];
        if (we > 0.0) {
          if (idx < 0 && tgt < run + we) {
            idx = i;
            lo = run;
          }
          last = i;
          lo_last = run;
        }
        run += we;
      }
      if (idx < 0) {
        idx = last;
        lo = lo_last;
      }
      sh.y = (int)((int64_t)tsel * kTile + (int64_t)owner * kUnit + idx);
      sh.lo = sh.off + ldexp(lo, e);
      sh.hi = sh.off + ldexp(lo + (double)sh.w8[idx], e);
    }
  }
  __syncthreads();
}

// pi(y)'s weight in draw units, with the precise residual (thread 0).
template <int DT, bool CUT = false, bool EPS = true>
__device__ double precise_weight(const VerifyArgs& a, int b, int k, int mode, const SampleCoef& cf, int y,
                                 const DrawLds& sh) {
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  const float lt = cut1<CUT>(load_one<DT>(trow, y), cf.Lt);
  const float ld = mode == kModeTarget ? 0.f : cut1<CUT>(load_one<DT>(drow, y), cf.Ld);
  SampleCoef c = cf;
  if (mode == kModeTarget && k == a.gamma) c.Mt = (float)(sh.Mp + sh.e);   // the tile's offset
  float w = 0.f, r;
  with_mode<EPS>(mode, [&](auto m) { w = weight_one<DT, decltype(m)::value, true>(ld, lt, c, r); });
  return ldexp((double)w, sh.e);
}

// Recompute every tile sum of a sequence in `mode`, the residual or q_k (a
// zero Saguaro normaliser falls back to the residual, a zero residual mass to
// q_k, k < gamma, whose offset Mt is the record's; degenerate inputs only).
// One logit at a time, with the weights and order the rescan uses, so its
// per-lane fp32 sums match.
template <int DT, bool CUT = false>
__device__ void recompute_tiles(const VerifyArgs& a, int b, int k, int mode, const SampleCoef& cf,
                                DrawLds& sh) {
  uint64_t* tiles = a.tiles + (int64_t)b * a.ntile;
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  for (int t = 0; t < a.ntile; ++t) {
    const int64_t j0 = (int64_t)t * kTile + (int64_t)threadIdx.x * kUnit;
    float ws = 0.f;
#pragma unroll 1
    for (int e = 0; e < kUnit; ++e) {
      const int64_t j = j0 + e;
      float w = 0.f, rr;
      if (j < a.V) {
        const float lt = cut1<CUT>(load_one<DT>(trow, j), cf.Lt);
        if (mode == kModeResidual)
          w = weight_one<DT, kModeResidual, false>(cut1<CUT>(load_one<DT>(drow, j), cf.Ld), lt, cf, rr);
        else w = weight_one<DT, kModeTarget, false>(0.f, lt, cf, rr);
      }
      ws += w;
    }
    const double tw = block_sum((double)ws, sh.lds_d);
    if (threadIdx.x == 0) slot_put(tiles + t, tw);
  }
  if (threadIdx.x == 0) wait_mem();
  __syncthreads();
}

// The drawn token of a sequence: the 64-bit word at byte 8 of its count line,
// stored as a complement (0 = not drawn yet).
__device__ __forceinline__ uint64_t* drawn_slot(const VerifyArgs& a, int b) {
  return reinterpret_cast<uint64_t*>(a.flag + (int64_t)b * kFlagStride + 2);
}

// The draw at the stopping position: tile values, locate, rescan.  The token
// goes to the sequence's drawn slot, the diagnostics out.  Clears the tile and
// residual-sum slots once read.
template <int DT, bool VEC, bool CUT = false, bool EPS = true>
__device__ void draw_item(const VerifyArgs& a, int b, DrawLds& sh) {
  const int tid = threadIdx.x;
  const SeqRec rec = wait_rec<true>(a, b);
  if (!rec.valid) return;
  const int g = a.gamma, k = rec.k;
  uint64_t* tiles = a.tiles + (int64_t)b * a.ntile;
  const float epsS = rec.mode == kModeSaguaroEps ? eps_clamp(a, b, sh.lds_d) : 0.f;
  const SampleCoef cf = coef_of<CUT>(a, b, rec, epsS);
  int mode = rec.mode;
  for (int t = tid; t < a.ntile; t += kThreads) (void)poll(a, tiles + t);
  double rtot = 0.0;   // residual mass (relative to Mt) when it differs from the tile total
  if (mode == kModeSaguaro || mode == kModeSaguaroEps) {
    uint64_t* rs = (mode == kModeSaguaro ? a.rsum : a.mass) + (int64_t)b * a.nt;
    for (int i = tid; i < a.nt; i += kThreads) rtot += slot_value(poll(a, rs + i));
  }
  rtot = uni(block_sum(rtot, sh.lds_d));   // also orders the polls before the reads below

  const double u = (double)a.u_smp[(int64_t)b * (g + 1) + k];
  double target = 0.0, S = 0.0;
  if (tid == 0) sh.Mp = 0.0;
  // A zero Saguaro normaliser falls back to the residual, a zero residual mass
  // to q_k (degenerate inputs only); one pass per mode.
  if (mode == kModeTarget) tiles_to_linear(tiles, a.ntile, sh);   // the bonus draw
  for (;;) {
    S = uni(locate_tile(tiles, a.ntile, u, sh, target));
    target = uni(target);
    if (mode == kModeResidual) rtot = S;
    if (S > 0.0 || mode == kModeTarget) break;
    mode = mode == kModeResidual ? kModeTarget : kModeResidual;
    recompute_tiles<DT, CUT>(a, b, k, mode, cf, sh);
  }
  with_mode<EPS>(mode, [&](auto m) { rescan_tile<DT, VEC, decltype(m)::value, CUT>(a, b, k, cf, target, sh); });
  if (tid == 0) {
    const int y = sh.y;
    if (a.diag.resid_mass) a.diag.resid_mass[b] = k < g ? rtot / rec.Zt : 0.0;
    if (a.diag.token_prob) a.diag.token_prob[b] = precise_weight<DT, CUT, EPS>(a, b, k, mode, cf, y, sh) / S;
    if (a.diag.cdf_lo) a.diag.cdf_lo[b] = sh.lo / S;
    if (a.diag.cdf_hi) a.diag.cdf_hi[b] = sh.hi / S;
    st_dev_u64(drawn_slot(a, b), ~(uint64_t)(uint32_t)y);
  }
  // Every tile and residual-sum slot of the sequence has been read.
  __syncthreads();
  for (int t = tid; t < a.ntile; t += kThreads) slot_clear(tiles + t);
  if (rec.mode == kModeSaguaro)
    for (int i = tid; i < a.nt; i += kThreads) slot_clear(a.rsum + (int64_t)b * a.nt + i);
  if (rec.mode == kModeSaguaroEps)
    for (int i = tid; i < a.nt; i += kThreads) slot_clear(a.mass + (int64_t)b * a.nt + i);
}

// ---------------------------------------------------------------------------
// Final item: target row gamma, which only the bonus draw reads and which is
// therefore streamed last, is checked, and the outputs are written.

struct FinalLds {
  int ok, y;
};

template <int DT>
__device__ void final_item(const VerifyArgs& a, int b, FinalLds& sh) {
  const int tid = threadIdx.x;
  const int g = a.gamma, R = 2 * g + 1, r = 2 * g;
  const SeqRec rec = wait_rec<false>(a, b);
  if (tid < 16) {
    double M, z;
    float mr;
    merge_row(a, b, r, tid, M, z, mr);
    if (tid == 0) {
      const bool ok = row_ok(M, z);
      sh.ok = ok;
      const bool read = !a.early || (rec.valid && rec.k == g);
      if (ok && read && a.diag.row_max) a.diag.row_max[(int64_t)b * R + r] = (double)mr * temp_coef(a, b).invT;
      if (ok && read && a.diag.row_logZ) a.diag.row_logZ[(int64_t)b * R + r] = M * 0.69314718055994530942 + log(z);
      if (rec.valid) {
        uint64_t* ys = drawn_slot(a, b);
        sh.y = (int)(uint32_t)~poll(a, ys);
        slot_clear(ys);
      }
    }
  }
  __syncthreads();
  if (rec.valid) {   // an invalid decision wrote its outputs already
    const int k = rec.k;
    if (!sh.ok && (!a.early || k == g)) {   // early exit reads target row gamma only for the bonus
      write_invalid(a, b, tid);
    } else {
      const int64_t orow = (int64_t)b * (g + 1);
      if (tid <= g) {
        int tok = -1;
        if (tid < k) tok = a.tokens[(int64_t)b * g + tid];
        else if (tid == k) tok = sh.y;
        a.out_tokens[orow + tid] = tok;
      }
      if (tid == 0) {
        a.out_acc[b] = k;
        if (a.out_first_reject) a.out_first_reject[b] = k < g ? k : -1;
        if (a.out_mask) a.out_mask[b] = rec.mask;
        if (a.out_len) a.out_len[b] = (a.in_len ? a.in_len[b] : 0) + k + 1;
      }
    }
  }
  // Once every other item of the sequence is done with the decision record,
  // clear it and the count.
  if (tid == 0) {
    unsigned* f = a.flag + (int64_t)b * kFlagStride;
    const unsigned expect = (unsigned)a.nt * ((a.saguaro && a.eps > 0.f) ? 2u : 1u) + 1u;
    unsigned polls = 0;
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < expect &&
           !give_up(a, polls)) {
    }
    if (a.early) {   // every position test has read the stop and progress words
      while (ld_dev_u32(f + kTestsWord) < (unsigned)g && !give_up(a, polls)) {
      }
      slot_clear32(f + kStopWord);
      slot_clear32(f + kProgWord);
      slot_clear32(f + kTestsWord);
    }
    slot_clear32(f);
    clear_rec(a.seq + b);
  }
}

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

// Two decoders of a block number: a binary search over the steps (the
// default order measures faster with it) and the segment table (the
// early-exit order, whose many short items gain from the shorter decode).
__device__ inline int64_t sched_offset_dev(const Sched& s, int t) {
  int64_t o = 0;
#pragma unroll
  for (int i = 0; i < kKinds; ++i) {
    int n = t - s.lag[i];
    n = n < 0 ? 0 : (n > s.count[i] ? s.count[i] : n);
    o += (int64_t)n * s.size[i];
  }
  return o;
}
__device__ inline void sched_decode_search(const Sched& s, int j, int& kind, int& b, int& sub) {
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
// Every index into the table is a constant (unrolled loops and selects), so
// the table is read straight from the kernel arguments.
__device__ inline void sched_decode_table(const Sched& s, int j, int& kind, int& b, int& sub) {
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

// ---------------------------------------------------------------------------
// Kernels.

union ItemLds {
  StreamLds s;
  DecideLds d;
  DrawLds r;
  FinalLds f;
  TestLds t;
};

// Early exit: a stream item of position pos (1..gamma-1) skips its rows when
// an earlier position is known to stop the sequence; an item of target row
// gamma (pos = gamma) skips on any known stop.  Read by one thread; the
// work-group follows its answer.
__device__ __forceinline__ bool early_stopped(const VerifyArgs& a, int b, int pos) {
  const unsigned st = ld_dev_u32(a.flag + (int64_t)b * kFlagStride + kStopWord);
  return pos >= a.gamma ? st != 0u : st > 64u - (unsigned)pos;
}
// A skipping item publishes skip markers in place of its piece.
__device__ __forceinline__ void early_skip(const VerifyArgs& a, int b, int r, int c) {
  if (threadIdx.x == 0) {
    const int64_t idx = ((int64_t)b * (2 * a.gamma + 1) + r) * a.nc + c;
    __hip_atomic_store(a.mraw + idx, kSkipRaw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st_dev_u64(a.part + idx, kSkipPiece);
  }
}

// Compiled for 8 waves per SIMD (64 VGPRs): the stream items need the
// occupancy; every other path fits without spilling for packed bf16 rows.
// PRED: outcome prediction too (draft-row items record lane leaders; the
// items of target row gamma are followed by leader items of draft row gamma).
// EARLY: the early-exit order (position-major stream items, position tests).
template <int DT, bool VEC, int U, bool PRED, bool EARLY>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void fused_kernel(VerifyArgs a, Sched sc) {
  __shared__ ItemLds sh;
  __shared__ int item[4];
  // One wave decodes the block number (a search on the scalar unit, which
  // the CU's waves share) and hands the item to the others.
  if (threadIdx.x < 64) {
    int kind, b, sub;
    if constexpr (EARLY) sched_decode_table(sc, (int)blockIdx.x, kind, b, sub);
    else sched_decode_search(sc, (int)blockIdx.x, kind, b, sub);
    if (threadIdx.x == 0) {
      item[0] = kind;
      item[1] = b;
      item[2] = sub;
      bool skip = false;
      if constexpr (EARLY) {
        if (kind == kItemStream && b >= a.B) skip = early_stopped(a, b - b / a.B * a.B, b / a.B);
        else if (kind == kItemLast) skip = early_stopped(a, b, a.gamma);
      }
      item[3] = skip;
    }
  }
  __syncthreads();
  const int kind = uni(item[0]), b = uni(item[1]), sub = uni(item[2]), skip = uni(item[3]);
  switch (kind) {
    case kItemStream: {
      if constexpr (EARLY) {   // b = i * B + sequence; sub: draft row i, then target row i
        const int i = b / a.B, q = b - i * a.B;
        const int h = sub >= a.nc, c = sub - h * a.nc, r = h ? a.gamma + i : i;
        if (skip) early_skip(a, q, r, c);
        else stream_item<DT, VEC, U>(a, q, r, c, sh.s);
      } else {
        const int r = sub / a.nc, c = sub - r * a.nc;
        if (PRED && r < a.gamma) stream_item<DT, VEC, U, PRED>(a, b, r, c, sh.s);
        else stream_item<DT, VEC, U>(a, b, r, c, sh.s);
      }
      break;
    }
    case kItemTest:
      if constexpr (EARLY) test_item<DT>(a, b - b / a.B * a.B, b / a.B, sh.t);
      break;
    case kItemDecide: decide_item<DT>(a, b, sh.d); break;
    case kItemMass: break;   // Saguaro with eps > 0 runs as separate kernels
    case kItemSample: sample_item<DT, VEC, false, false>(a, b, sub, sh.r.lds_d); break;
    case kItemDraw: draw_item<DT, VEC, false, false>(a, b, sh.r); break;
    case kItemLast:
      if (EARLY && skip) {
        early_skip(a, b, 2 * a.gamma, sub);
        break;
      }
      if (!PRED || sub < a.nc) stream_item<DT, VEC, U>(a, b, 2 * a.gamma, sub, sh.s);
      else leader_item<DT, VEC, U>(a, b, sub - a.nc, sh.s);
      break;
    default: final_item<DT>(a, b, sh.f); break;
  }
}

template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kThreads) void stream_kernel(VerifyArgs a) {
  __shared__ StreamLds sh;
  const int R = 2 * a.gamma + 1;
  const int64_t id = blockIdx.x;
  const int per_seq = R * a.nc;
  const int b = (int)(id / per_seq);
  const int rem = (int)(id - (int64_t)b * per_seq);
  const int r = rem / a.nc, c = rem - r * a.nc;
  stream_item<DT, VEC, U>(a, b, r, c, sh);
}

template <int DT, bool CUT>
__global__ __launch_bounds__(kThreads) void decide_kernel(VerifyArgs a) {
  __shared__ DecideLds sh;
  decide_item<DT, CUT>(a, blockIdx.x, sh);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void test_kernel(VerifyArgs a) {
  __shared__ TestLds sh;
  const int i = blockIdx.x / a.B;
  test_item<DT>(a, blockIdx.x - i * a.B, i, sh);
}

template <int DT, bool VEC, bool CUT>
__global__ __launch_bounds__(kThreads) void mass_kernel(VerifyArgs a) {
  __shared__ double lds_d[kWaves * (kTilesPerItem + 1)];
  const int b = blockIdx.x / a.nt, s = blockIdx.x - b * a.nt;
  mass_item<DT, VEC, CUT>(a, b, s, lds_d);
}

template <int DT, bool VEC, bool CUT>
__global__ __launch_bounds__(kThreads) void sample_kernel(VerifyArgs a) {
  __shared__ double lds_d[kWaves * (kTilesPerItem + 1)];
  const int b = blockIdx.x / a.nt, s = blockIdx.x - b * a.nt;
  sample_item<DT, VEC, CUT>(a, b, s, lds_d);
}

template <int DT, bool VEC, bool CUT>
__global__ __launch_bounds__(kThreads) void draw_kernel(VerifyArgs a) {
  __shared__ DrawLds sh;
  draw_item<DT, VEC, CUT>(a, blockIdx.x, sh);
}

// ---------------------------------------------------------------------------
// Top-p: the nucleus threshold of every row by a radix selection over the
// logits' order-preserving keys (16 bits for bfloat16, 32 for float32; 8 bits
// a pass), each key weighted by its probability mass, from the highest key
// down, until the mass reaches top_p.

// The order-preserving key of a logit (+0.0 and -0.0 share one), in kb bits.
template <int DT>
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return DT == kBF16 ? k >> 16 : k;
}
template <int DT>
__device__ __forceinline__ float key_logit(uint32_t k) {
  if constexpr (DT == kBF16) {
    const uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    return __uint_as_float(b << 16);
  } else {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  }
}

// One wave per row: the row's offset and normaliser from its pieces (left in
// place for the decision), and the selection's start.
__global__ __launch_bounds__(64) void topp_init_kernel(VerifyArgs a) {
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t* p = a.part + row * a.nc;
  double M = -INFINITY;
  for (int c = lane; c < a.nc; c += 64) M = fmax(M, slot_value(ld_dev_u64(p + c)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmax(M, __shfl_xor(M, o, 64));
  M = ceil(M);
  double z = 0.0;
  for (int c = lane; c < a.nc; c += 64) {
    const double v = slot_value(ld_dev_u64(p + c));
    if (v != -INFINITY) z += exp2(v - M);
  }
  z = wave_sum(z);
  if (lane == 0) {
    TopPRow t;
    t.M = M;
    t.Z = z;
    t.rem = (double)a.top_p * z;
    t.above = 0.0;
    t.P = 1.0;
    t.prefix = 0u;
    t.L = -INFINITY;
    a.topp[row] = t;
  }
}

// (row, chunk) items: the masses of the chunk's logits whose key matches the
// selected prefix, by the pass's digit, into the row's histogram.  Each wave
// has its own LDS histogram (fewer colliding atomics); a lane sums runs of
// one digit before adding.  Loads: four units in flight per lane.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void topp_hist_kernel(VerifyArgs a, int pass) {
  __shared__ double h[kWaves][kDigits];
  const int R = 2 * a.gamma + 1;
  const int64_t id = blockIdx.x;
  const int64_t row = id / a.nc;
  const int c = (int)(id - row * a.nc);
  const int b = (int)(row / R), r = (int)(row - (int64_t)b * R);
  const TCoef tc = temp_coef(a, b);
  const float Mf = (float)uni(a.topp[row].M);
  const uint32_t prefix = (uint32_t)uni((int)a.topp[row].prefix);
  constexpr int KB = DT == kBF16 ? 16 : 32;
  const int shift = KB - 8 * (pass + 1);
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWaves * kDigits; i += kThreads) (&h[0][0])[i] = 0.0;
  __syncthreads();
  const void* rp = row_ptr<DT>(a, b, r);
  const int64_t begin = (int64_t)c * a.chunk;
  const int64_t end = min<int64_t>(begin + a.chunk, a.V);
  int cur = -1;
  double acc = 0.0;
  auto take = [&](const Raw8<DT, VEC>& raw, int64_t j) {
    float v[8];
    unpack<DT, VEC>(raw, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (j + e >= end) continue;
      const uint32_t key = logit_key<DT>(v[e]);
      if (pass > 0 && (key >> (shift + 8)) != prefix) continue;
      const int d = (int)((key >> shift) & 0xFFu);
      const double m = (double)exp2_fast(fmaf(v[e], tc.c_lo, fmaf(v[e], tc.c_hi, -Mf)));
      if (d != cur) {
        if (cur >= 0) atomicAdd(&h[wave][cur], acc);
        cur = d;
        acc = 0.0;
      }
      acc += m;
    }
  };
  constexpr int U = 4;
  int64_t j = begin + (int64_t)threadIdx.x * kUnit;
  for (; j + (U - 1) * (int64_t)kTile < end; j += U * (int64_t)kTile) {
    Raw8<DT, VEC> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load_raw<DT, VEC, true>(rp, j + u * (int64_t)kTile, end, raw[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) take(raw[u], j + u * (int64_t)kTile);
  }
  for (; j < end; j += kTile) {
    Raw8<DT, VEC> raw;
    load_raw<DT, VEC, true>(rp, j, end, raw);
    take(raw, j);
  }
  if (cur >= 0) atomicAdd(&h[wave][cur], acc);
  __syncthreads();
  double* g = a.hist + row * kDigits;
  for (int i = threadIdx.x; i < kDigits; i += kThreads) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += h[w][i];
    if (t != 0.0) atomicAdd(g + i, t);
  }
}

// One wave per row: the digit at which the mass from the top reaches the
// remaining target; clears the histogram.  Lane l holds digits 4l..4l+3 and
// a suffix sum over the lanes gives the mass above each lane's digits.  If
// rounding left the target above the row's total, every digit is kept (the
// lowest digit with mass is selected).  After the last pass, the threshold
// logit and the nucleus mass.
template <int DT>
__global__ __launch_bounds__(64) void topp_select_kernel(VerifyArgs a, int pass, int npass) {
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  TopPRow t = a.topp[row];
  double* g = a.hist + row * kDigits;
  double m[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) m[q] = g[4 * lane + q];
#pragma unroll
  for (int q = 0; q < 4; ++q) g[4 * lane + q] = 0.0;
  const double mine = (m[0] + m[1]) + (m[2] + m[3]);
  double incl = mine;   // inclusive suffix sum over the lanes (higher digits)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double x = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += x;
  }
  const double above_lane = incl - mine;
  // In this lane, from its highest digit down: the first that reaches the target.
  int sel = -1;
  double run = above_lane, hsel = 0.0, before = 0.0;
#pragma unroll
  for (int q = 3; q >= 0; --q) {
    if (sel < 0 && m[q] > 0.0 && run + m[q] >= t.rem) {
      sel = 4 * lane + q;
      hsel = m[q];
      before = run;
    }
    if (sel < 0) run += m[q];
  }
  // The lowest digit with mass in this lane, for the keep-everything case.
  int low = -1;
  double low_h = 0.0, low_before = 0.0;
  {
    double r2 = above_lane;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      if (m[q] > 0.0) {
        low = 4 * lane + q;
        low_h = m[q];
        low_before = r2;
      }
      r2 += m[q];
    }
  }
  const uint64_t has = __ballot(sel >= 0);
  const uint64_t haslow = __ballot(low >= 0);
  int src, s_sel;
  double s_h, s_before;
  if (has) {   // the highest digit (lane) that reaches the target
    src = 63 - __builtin_clzll(has);
    s_sel = __shfl(sel, src, 64);
    s_h = __shfl(hsel, src, 64);
    s_before = __shfl(before, src, 64);
  } else {     // keep everything down to the lowest digit with mass
    src = haslow ? __builtin_ctzll(haslow) : 0;
    s_sel = haslow ? __shfl(low, src, 64) : 0;
    s_h = haslow ? __shfl(low_h, src, 64) : 0.0;
    s_before = haslow ? __shfl(low_before, src, 64) : 0.0;
  }
  if (lane == 0) {
    t.above += s_before;
    t.rem -= s_before;
    t.prefix = (t.prefix << 8) | (uint32_t)s_sel;
    if (pass == npass - 1) {
      t.L = key_logit<DT>(t.prefix);
      t.P = (t.above + s_h) / t.Z;
    }
    a.topp[row] = t;
  }
}


// Top-p of bfloat16 rows by counting.  A bfloat16 row holds at most 65536
// distinct values and every logit of one value carries the same mass, so the
// row's masses in value order follow exactly from how often each value
// occurs.  One 1024-thread work-group per row:
//   * counts the row's values by their 16-bit order-preserving keys in LDS,
//     two 16-bit counters per 32-bit word: word w counts key w (a negative
//     value) in its low half and key w + 32768 (a non-negative one) in its
//     high half, so neighbouring values, which a row's logits crowd, fall in
//     different words.  A counter wraps only where one value occurs 65536
//     times or more; the counters then sum to less than V, and the row is
//     counted again with returning atomics that record every wrap, so only
//     such rows are read twice;
//   * from the counts, from the top key down: the largest finite value (the
//     row offset), the row normaliser in fp64, and the nucleus threshold (the
//     first value at whose end the running mass reaches top_p times the
//     normaliser; each value is one run of equal logits);
//   * writes the row's normaliser piece (the whole row in piece 0, -inf in
//     the others) and its maximum where the stream items would, so a cut
//     bfloat16 row needs no stream items.
constexpr int kCountThreads = 1024;
constexpr int kCountWaves = kCountThreads / 64;
constexpr int kCountWords = 32768;                                     // 128 KB of counters
constexpr int kWordsPerThread = kCountWords / kCountThreads;           // 32
// Wraps in a row of V logits: at most V / 65536 of low counters, plus
// (V + those) / 65536 of high counters (each low wrap carries one into the
// high counter of its word): at most 256 up to this row length.  Longer
// bfloat16 rows take the radix selection.
constexpr int64_t kCountMaxV = (int64_t)1 << 24;
constexpr int kCountEvents = 288;
constexpr uint32_t kKeyNegInf = 0x007Fu, kKeyNegZero = 0x7FFFu, kKeyPosZero = 0x8000u,
                   kKeyPosInf = 0xFF80u;

// The counted row's words with a count, compacted in ascending order (word,
// low count | high count << 16) for the wave that finishes the row while the
// next one is counted; a row with more takes the in-place finish.
constexpr int kListCap = 3328;
constexpr int kCountingWaves = kCountWaves - 1;
constexpr int kCountingThreads = 64 * kCountingWaves;

struct CountLds {
  uint32_t cnt[kCountWords];
  uint2 list[kListCap];
  uint32_t ev[kCountEvents];   // keys whose counter wrapped (checked pass)
  uint32_t nev;
  uint32_t sum[kCountWaves], nzw[kCountWaves];
  int kmax[kCountWaves], flags[kCountWaves];
  double tot[2][kCountWaves];
  int sel;
  double P;
};

// The keys of the two bfloat16 logits in w (its halves), in the halves of
// the result: a negative value's bits inverted, a non-negative value's sign
// bit set.  -0 takes key 0x7FFF, next below +0's 0x8000; both are the value
// zero and are merged when the counts are read.
__device__ __forceinline__ uint32_t bf16_key_pair(uint32_t w) {
  const uint32_t s = w & 0x80008000u;
  return w ^ (0x80008000u | (s - (s >> 15)));
}

__device__ __forceinline__ void count_wrap(CountLds& sh, uint32_t k) {
  const uint32_t e = __hip_atomic_fetch_add(&sh.nev, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (e < (uint32_t)kCountEvents) sh.ev[e] = k;
}

// CHECK: the atomic returns the old word, and a counter that was 0xFFFF has
// wrapped (a low one carrying into the high one, which may wrap in turn).
template <bool CHECK>
__device__ __forceinline__ void count_key(CountLds& sh, uint32_t k) {
  const uint32_t inc = (k >> 15) * 0xFFFFu + 1u;
  uint32_t* w = sh.cnt + (k & 0x7FFFu);
  if constexpr (!CHECK) {
    __hip_atomic_fetch_add(w, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    const uint32_t old = __hip_atomic_fetch_add(w, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t lo = old & 0xFFFFu, hi = old >> 16;
    if ((k >> 15) ? hi == 0xFFFFu : lo == 0xFFFFu) {
      count_wrap(sh, k);
      if (!(k >> 15) && hi == 0xFFFFu) count_wrap(sh, k + 32768u);
    }
  }
}
template <bool CHECK>
__device__ __forceinline__ void count_pair(CountLds& sh, uint32_t w) {
  const uint32_t kp = bf16_key_pair(w);
  count_key<CHECK>(sh, kp & 0xFFFFu);
  count_key<CHECK>(sh, kp >> 16);
}

// Every logit of the row, once, by threads 0 .. NT - 1.  Lane t takes
// 8-logit units t, t + NT, ... (eight in flight; one in the rarely run
// checked pass, whose code stays small), then one of the last V mod 8.
template <bool VEC, bool CHECK, int NT>
__device__ void count_row(const uint16_t* row, int64_t V, CountLds& sh) {
  const int t = threadIdx.x;
  const int64_t units = V >> 3;
  int64_t u = t;
  if constexpr (VEC) {
    constexpr int U = CHECK ? 1 : 8;
    constexpr int64_t kBatch = (int64_t)U * NT;
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(row, (int)(units * 16));
    const int voff = t * 16;
    const int64_t nb = units / kBatch;
    for (int64_t i = 0; i < nb; ++i) {
      u32x4 w[U];
#pragma unroll
      for (int q = 0; q < U; ++q)
        w[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (int)((i * kBatch + q * NT) * 16), 2);
#pragma unroll
      for (int q = 0; q < U; ++q) {
        count_pair<CHECK>(sh, w[q].x);
        count_pair<CHECK>(sh, w[q].y);
        count_pair<CHECK>(sh, w[q].z);
        count_pair<CHECK>(sh, w[q].w);
      }
    }
    for (u = nb * kBatch + t; u < units; u += NT) {
      const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (int)((u - t) * 16), 2);
      count_pair<CHECK>(sh, w.x);
      count_pair<CHECK>(sh, w.y);
      count_pair<CHECK>(sh, w.z);
      count_pair<CHECK>(sh, w.w);
    }
  } else {
    for (; u < units; u += NT) {
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        count_pair<CHECK>(sh, (uint32_t)row[u * 8 + e] | ((uint32_t)row[u * 8 + e + 1] << 16));
    }
  }
  if (t < V - units * 8) count_key<CHECK>(sh, bf16_key_pair(row[units * 8 + t]) & 0xFFFFu);
}

__device__ __forceinline__ bool key_finite(uint32_t k) { return k > kKeyNegInf && k < kKeyPosInf; }
// Flags of a key outside the finite range: 1 for a NaN, 2 for +inf, 0 for -inf.
__device__ __forceinline__ int nonfinite_flag(uint32_t k) {
  return k == kKeyNegInf ? 0 : (k == kKeyPosInf ? 2 : 1);
}

// The count of key k from its 16-bit counter and the recorded wraps: 65536
// more per wrap of k, one less per carry into k (a wrap of the low counter
// of k's word, when k is the high one).
__device__ __forceinline__ uint32_t key_count(const CountLds& sh, int nev, uint32_t k) {
  uint32_t h = (sh.cnt[k & 0x7FFFu] >> (16 * (k >> 15))) & 0xFFFFu;
  for (int e = 0; e < nev; ++e) {
    const uint32_t x = sh.ev[e];
    if (x == k) h += 65536u;
    else if ((k >> 15) && x == k - 32768u) h -= 1u;
  }
  return h;
}

// Inclusive suffix sum over the lanes of a wave (lane 63 first).
template <typename F>
__device__ __forceinline__ F wave_suffix_sum(F v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const F y = __shfl_down(v, o, 64);
    if (lane + o < 64) v += y;
  }
  return v;
}

// A counted row's outputs: its normaliser piece (the whole row in piece 0,
// -inf in the others) and maximum where the stream items would put them,
// and its nucleus (threshold sel, mass fraction P; none for a bad row).
// Threads tid = 0 .. nthr - 1.
__device__ __forceinline__ void count_outputs(const VerifyArgs& a, int64_t row, int flags, int kmax, float mref,
                                              double Z, int sel, double P, int tid, int nthr) {
  const bool bad = flags != 0 || kmax < 0;
  const float vmax = kmax >= 0 ? key_logit<kBF16>((uint32_t)kmax) : -INFINITY;
  const int64_t p0 = row * a.nc;
  for (int i = tid; i < a.nc; i += nthr) {
    double v = -INFINITY;
    float mr = -INFINITY;
    if (i == 0) {
      if (flags & 1) v = NAN;
      else if (flags & 2) v = INFINITY;
      else if (kmax >= 0) v = (double)mref + log2(Z);
      mr = (flags & 2) ? INFINITY : vmax;
    }
    slot_put32(a.mraw + p0 + i, mr);
    slot_put(a.part + p0 + i, v);
  }
  if (tid == 0) {
    TopPRow tr;
    tr.M = mref;
    tr.Z = Z;
    tr.rem = 0.0;
    tr.above = 0.0;
    const bool cut = !bad && sel >= 0;
    tr.P = cut ? P : 1.0;
    tr.prefix = cut ? (uint32_t)sel : 0u;
    tr.L = cut ? key_logit<kBF16>((uint32_t)sel) : -INFINITY;
    a.topp[row] = tr;
  }
}

// The in-place finish of a counted row (every thread): wave w takes words
// 2048w + 64j + lane (j = 0..31) in registers, consecutive words in
// consecutive lanes, so a band of crowded values spreads over the lanes.
// From the top key down the order is: the high halves (non-negative values)
// of waves 15..0, then the low halves of waves 15..0; within a wave, rows
// j = 31..0, lanes 63..0.  Leaves counts in the counters.
template <bool VEC>
__device__ void finish_inplace(const VerifyArgs& a, int64_t row, CountLds& sh) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int R = 2 * a.gamma + 1;
  const int b = (int)(row / R), r = (int)(row - (int64_t)b * R);
  const uint16_t* rp = static_cast<const uint16_t*>(row_ptr<kBF16>(a, b, r));
  const TCoef tc = temp_coef(a, b);
  uint4* c4 = reinterpret_cast<uint4*>(sh.cnt);

  // Word of row j: wbase + 64 j (the opaque step keeps the compiler from
  // precomputing every such address outside the caller's loop).
  uint32_t wbase = 2048u * (uint32_t)wave + (uint32_t)lane;
  asm volatile("" : "+v"(wbase));
  // The counter words are read from LDS where used (rare path: registers
  // stay free).
  auto cw = [&](int j) -> uint32_t { return sh.cnt[wbase + 64u * j]; };
  int nev = 0;
  {   // the 16-bit counters sum to V unless one wrapped: then count again, recording the wraps
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) sum += (cw(j) & 0xFFFFu) + (cw(j) >> 16);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) sh.sum[wave] = sum;
    __syncthreads();
    sum = 0;
    for (int i = 0; i < kCountWaves; ++i) sum += sh.sum[i];
    if ((int64_t)sum != a.V) {
      __syncthreads();   // every thread is done with the counters
      for (int i = t; i < kCountWords / 4; i += kCountThreads) c4[i] = make_uint4(0u, 0u, 0u, 0u);
      if (t == 0) sh.nev = 0u;
      __syncthreads();
      count_row<VEC, true, kCountThreads>(rp, a.V, sh);
      __syncthreads();
      nev = (int)min(sh.nev, (uint32_t)kCountEvents);
    }
  }
  // The count of key half h of row j (with the recorded wraps, if any); -0
  // counts with +0 (key 0x8000, the high half of word 0).
  const uint32_t nzero = key_count(sh, nev, kKeyNegZero);
  auto count_at = [&](int j, int h) -> uint32_t {
    const uint32_t k = wbase + 64u * j + 32768u * h;
    uint32_t n = nev ? key_count(sh, nev, k) : ((cw(j) >> (16 * h)) & 0xFFFFu);
    return k == kKeyNegZero ? 0u : (k == kKeyPosZero ? n + nzero : n);
  };

  // The largest finite key with a count, and flags (1: a NaN, 2: +inf).
  // Keys outside the finite range: the low halves of words 0..127 (wave 0,
  // rows 0 and 1) and the high halves of words 32640..32767 (wave 15, rows
  // 30 and 31).
  int kmax = -1, flags = 0;
  auto take = [&](uint32_t k, uint32_t n) {
    const bool fin = key_finite(k);
    kmax = (n != 0u && fin) ? max(kmax, (int)k) : kmax;
    flags |= (n != 0u && !fin) ? nonfinite_flag(k) : 0;
  };
  if (nev == 0) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t w = cw(j);
      asm volatile("" : "+v"(w), "+v"(kmax), "+v"(flags));
      const uint32_t k = wbase + 64u * j;
      take(k, k == kKeyNegZero ? 0u : (w & 0xFFFFu));
      take(k + 32768u, k == 0u ? (w >> 16) + nzero : (w >> 16));
    }
  } else {
    for (uint32_t j = 0; j < 32u; ++j)
      for (uint32_t h = 0; h < 2u; ++h) {
        const uint32_t k = wbase + 64u * j + 32768u * h;
        const uint32_t n = key_count(sh, nev, k);
        take(k, k == kKeyNegZero ? 0u : (k == kKeyPosZero ? n + nzero : n));
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmax = max(kmax, __shfl_xor(kmax, o, 64));
    flags |= __shfl_xor(flags, o, 64);
  }
  if (lane == 0) {
    sh.kmax[wave] = kmax;
    sh.flags[wave] = flags;
  }
  __syncthreads();
  for (int i = 0; i < kCountWaves; ++i) {
    kmax = max(kmax, sh.kmax[i]);
    flags |= sh.flags[i];
  }

  // Masses count * 2^(l c_T - mref) (0 for no count or a key outside the
  // finite range): each wave's sums over its high and low halves, in fp64.
  const bool bad = flags != 0 || kmax < 0;
  const float vmax = kmax >= 0 ? key_logit<kBF16>((uint32_t)kmax) : -INFINITY;
  const float mref = bad ? 0.f : ceilf(fminf(vmax * tc.c_hi, 1.0e30f));
  auto mass = [&](uint32_t k, uint32_t n) -> float {
    const float v = key_logit<kBF16>(k);
    const float m = (float)n * exp2_fast(fmaf(v, tc.c_lo, fmaf(v, tc.c_hi, -mref)));
    return (n != 0u && key_finite(k)) ? m : 0.f;
  };
  double cs[2] = {0.0, 0.0};
  if (!bad) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      // One row at a time (the opaque step orders them): computing every
      // term ahead of the additions would not fit the registers.
      uint32_t w = cw(j);
      asm volatile("" : "+v"(w), "+v"(cs[0]), "+v"(cs[1]));
      if (w != 0u || nev != 0 || (t == 0 && j == 0)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) cs[h] += (double)mass(wbase + 64u * j + 32768u * h, count_at(j, h));
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const double wt = wave_sum(cs[h]);
    if (lane == 0) sh.tot[h][wave] = wt;
  }
  if (t == 0) sh.sel = -1;
  __syncthreads();

  // Running sums over the 32 (half, wave) blocks from the top, the same
  // additions in the same order in every thread: Z, and the first block at
  // whose end the sum reaches top_p * Z (ab: the sum before it).
  double Z = 0.0;
  for (int i = 2 * kCountWaves - 1; i >= 0; --i) Z = Z + sh.tot[i / kCountWaves][i % kCountWaves];
  const double tgt = (double)a.top_p * Z;
  double ab = 0.0;
  int hx = -1, wx = -1;
  {
    double run = 0.0;
    for (int i = 2 * kCountWaves - 1; i >= 0 && hx < 0; --i) {
      const double bt = sh.tot[i / kCountWaves][i % kCountWaves], nx = run + bt;
      if (bt > 0.0 && nx >= tgt) {
        hx = i / kCountWaves;
        wx = i % kCountWaves;
        ab = run;
      }
      run = nx;
    }
  }
  if (!bad && wave == wx) {
    // The rows' sums of half hx over the lanes: a butterfly that halves the
    // rows each lane carries at every step leaves row lane / 2 in lanes
    // 2j and 2j + 1.
    float m[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) m[j] = mass(wbase + 64u * j + 32768u * hx, count_at(j, hx));
#pragma unroll
    for (int step = 0; step < 5; ++step) {
      const int half = 16 >> step, o = 32 >> step;
      const bool up = (lane & o) != 0;
#pragma unroll
      for (int k = 0; k < half; ++k) {
        const float send = up ? m[k] : m[k + half];
        const float recv = __shfl_xor(send, o, 64);
        m[k] = (up ? m[k + half] : m[k]) + recv;
      }
    }
    const float rj = m[0] + __shfl_xor(m[0], 1, 64);   // row lane / 2
    // Suffix sums over the rows (row 31 first): lane 2j holds rows >= j.
    const double sj = wave_suffix_sum((lane & 1) ? 0.0 : (double)rj, lane);
    const double incl = ab + sj;
    const double nxt = __shfl_down(sj, 2, 64);
    const double above = lane >= 62 ? ab : ab + nxt;
    const uint64_t crossr = __ballot(!(lane & 1) && rj > 0.f && above < tgt && tgt <= incl);
    const uint64_t hasr = __ballot(!(lane & 1) && rj > 0.f);
    // The crossing row; rounding aside (the rows' sums and the block's
    // differ in order), else the lowest row with mass.
    const int jl = crossr ? (63 - __builtin_clzll(crossr)) : __builtin_ctzll(hasr);
    const int jx = jl >> 1;
    const double ab_row = __shfl(above, jl, 64);
    // Keys of row jx, one per lane: the highest with mass whose running sum
    // reaches the target ends the nucleus (else the lowest with mass).
    const uint32_t k = wbase + 64u * (uint32_t)jx + 32768u * (uint32_t)hx;
    uint32_t n = nev ? key_count(sh, nev, k) : ((sh.cnt[k & 0x7FFFu] >> (16 * hx)) & 0xFFFFu);
    n = k == kKeyNegZero ? 0u : (k == kKeyPosZero ? n + nzero : n);
    const float mk = mass(k, n);
    const double run = wave_suffix_sum((double)mk, lane) + ab_row;
    const uint64_t hit = __ballot(mk != 0.f && run >= tgt);
    const uint64_t has = __ballot(mk != 0.f);
    const int src = hit ? 63 - __builtin_clzll(hit) : __builtin_ctzll(has);
    if (lane == src) {
      sh.sel = (int)k;
      sh.P = run / Z;
    }
  }
  __syncthreads();
  count_outputs(a, row, flags, kmax, mref, Z, sh.sel, sh.P, t, kCountThreads);
}

// The previous row's finish from its compacted words (one wave, while the
// other waves count the next row).  Lane l takes a run of consecutive
// entries; from the top key down the order is the high halves of entries
// E-1..0, then the low halves of entries E-1..0.  -0 has been counted with
// +0 already and no counter wrapped.
__device__ void finish_list(const VerifyArgs& a, int64_t row, const CountLds& sh, int E) {
  const int lane = threadIdx.x & 63;
  const int R = 2 * a.gamma + 1;
  const int b = (int)(row / R);
  const TCoef tc = temp_coef(a, b);
  const int per = (E + 63) >> 6;
  const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
  int kmax = -1, flags = 0;
  for (int e = e0; e < e1; ++e) {
    const uint2 en = sh.list[e];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t k = en.x + 32768u * h, n = (en.y >> (16 * h)) & 0xFFFFu;
      if (n == 0u) continue;
      if (key_finite(k)) kmax = max(kmax, (int)k);
      else flags |= nonfinite_flag(k);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmax = max(kmax, __shfl_xor(kmax, o, 64));
    flags |= __shfl_xor(flags, o, 64);
  }
  const bool bad = flags != 0 || kmax < 0;
  const float vmax = kmax >= 0 ? key_logit<kBF16>((uint32_t)kmax) : -INFINITY;
  const float mref = bad ? 0.f : ceilf(fminf(vmax * tc.c_hi, 1.0e30f));
  auto mass = [&](uint32_t k, uint32_t n) -> float {
    const float v = key_logit<kBF16>(k);
    const float m = (float)n * exp2_fast(fmaf(v, tc.c_lo, fmaf(v, tc.c_hi, -mref)));
    return (n != 0u && key_finite(k)) ? m : 0.f;
  };
  double sm[2] = {0.0, 0.0};
  if (!bad) {
    for (int e = e0; e < e1; ++e) {
      const uint2 en = sh.list[e];
      sm[0] += (double)mass(en.x, en.y & 0xFFFFu);
      sm[1] += (double)mass(en.x + 32768u, en.y >> 16);
    }
  }
  // Suffix sums over the lanes, the high halves first; a lane's `above` is
  // the next lane's `incl`, the same value, so the intervals tile (0, Z].
  const double s1 = wave_suffix_sum(sm[1], lane), s0 = wave_suffix_sum(sm[0], lane);
  const double H = __shfl(s1, 0, 64);
  const double d1 = __shfl_down(s1, 1, 64), d0 = __shfl_down(s0, 1, 64);
  const double incl1 = s1, above1 = lane == 63 ? 0.0 : d1;
  const double incl0 = s0 + H, above0 = (lane == 63 ? 0.0 : d0) + H;
  const double Z = __shfl(incl0, 0, 64);
  const double tgt = (double)a.top_p * Z;
  const bool c1 = !bad && above1 < tgt && tgt <= incl1, c0 = !bad && above0 < tgt && tgt <= incl0;
  int sel = -1;
  double P = 1.0;
  if (c1 || c0) {   // this lane's entries hold the threshold: walk them from the top
    const int h = c1 ? 1 : 0;
    double run = c1 ? above1 : above0, Pl = run;
    int low = -1;
    for (int e = e1 - 1; e >= e0; --e) {
      const uint2 en = sh.list[e];
      const uint32_t k = en.x + 32768u * h;
      const float m = mass(k, (en.y >> (16 * h)) & 0xFFFFu);
      if (m == 0.f) continue;
      run += (double)m;
      low = (int)k;
      Pl = run;
      if (run >= tgt) break;
    }
    sel = low;
    P = Pl / Z;
  }
  const uint64_t who = __ballot(sel >= 0);
  if (who) {
    const int src = __builtin_ctzll(who);
    sel = __shfl(sel, src, 64);
    P = __shfl(P, src, 64);
  }
  count_outputs(a, row, flags, kmax, mref, Z, sel, P, lane, 64);
}

// Persistent: work-group g counts rows g, g + G, ...  While waves 0..14
// count a row, wave 15 finishes the row before it from its compacted words
// (the counting is limited by LDS atomics, the finish by latency, so they
// overlap).  After each row every thread compacts its words with a count
// into the list and clears its counters; a row whose 16-bit counters
// wrapped, or whose words do not fit the list, is finished in place.
template <bool VEC>
__global__ __launch_bounds__(kCountThreads) void topp_count_kernel(VerifyArgs a, int64_t nrows) {
  __shared__ CountLds sh;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int R = 2 * a.gamma + 1;
  uint4* c4 = reinterpret_cast<uint4*>(sh.cnt);
  for (int i = t; i < kCountWords / 4; i += kCountThreads) c4[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  int64_t prev = -1;
  int E = 0;
  for (int64_t row = blockIdx.x;; row += gridDim.x) {
    const bool have = row < nrows;
    if (wave < kCountingWaves) {
      if (have) {
        const int b = (int)(row / R), r = (int)(row - (int64_t)b * R);
        count_row<VEC, false, kCountingThreads>(static_cast<const uint16_t*>(row_ptr<kBF16>(a, b, r)), a.V, sh);
      }
    } else if (prev >= 0) {
      finish_list(a, prev, sh, E);
    }
    __syncthreads();
    if (!have) break;

    // Compaction.  -0 (the low half of word 32767) moves to +0 (the high
    // half of word 0); the sum of the counters checks for a wrap.  Words
    // are read from LDS as needed (registers stay free for the counting);
    // word of row j: wbase + 64 j.
    uint32_t wbase = 2048u * (uint32_t)wave + (uint32_t)lane;
    asm volatile("" : "+v"(wbase));
    const uint32_t nzero = sh.cnt[kKeyNegZero] & 0xFFFFu;
    auto word = [&](int j) -> uint32_t {
      uint32_t w = sh.cnt[wbase + 64u * j];
      if (t == kCountThreads - 1 && j == 31) w &= 0xFFFF0000u;
      if (t == 0 && j == 0) w += nzero << 16;   // checked against overflow below
      return w;
    };
    uint32_t sum = 0, nzc = 0;
    int over = t == 0 && (sh.cnt[0] >> 16) + nzero > 0xFFFFu;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const uint32_t w = sh.cnt[wbase + 64u * j];
      sum += (w & 0xFFFFu) + (w >> 16);
      nzc += (uint32_t)__popcll(__ballot(word(j) != 0u));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    over = __ballot(over) != 0;
    if (lane == 0) {
      sh.sum[wave] = sum;
      sh.nzw[wave] = nzc;
      sh.flags[wave] = over;
    }
    __syncthreads();
    uint32_t tsum = 0, base = 0, tot = 0;
    for (int i = 0; i < kCountWaves; ++i) {
      tsum += sh.sum[i];
      base += i < wave ? sh.nzw[i] : 0u;
      tot += sh.nzw[i];
      over |= sh.flags[i];
    }
    if ((int64_t)tsum == a.V && tot <= (uint32_t)kListCap && !over) {
      // Each thread reads only its own words here (-0's counter was read
      // before the barrier above), so it clears each once read.
      const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll 8
      for (int j = 0; j < 32; ++j) {
        const uint32_t w = word(j);
        sh.cnt[wbase + 64u * j] = 0u;
        const uint64_t bal = __ballot(w != 0u);
        if (w != 0u) sh.list[base + (uint32_t)__popcll(bal & lt)] = make_uint2(wbase + 64u * j, w);
        base += (uint32_t)__popcll(bal);
      }
      prev = row;
      E = (int)tot;
    } else {
      finish_inplace<VEC>(a, row, sh);
      __syncthreads();
      for (int i = t; i < kCountWords / 4; i += kCountThreads) c4[i] = make_uint4(0u, 0u, 0u, 0u);
      prev = -1;
    }
    __syncthreads();
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void final_kernel(VerifyArgs a) {
  __shared__ FinalLds sh;
  final_item<DT>(a, blockIdx.x, sh);
}

// ---------------------------------------------------------------------------
// Host side.

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  int nc, chunk, ntile, nt;
  size_t err_off, part_off, mraw_off, seq_off, flag_off, tiles_off, mass_off, rsum_off, cpart_off,
      topp_off, hist_off, total;
};

static bool sizes_ok(int B, int gamma, int V) {
  return B >= 0 && gamma >= 1 && gamma <= 63 && V >= 1;
}

static Layout layout(int B, int gamma, int V) {
  Layout L;
  // Chunks are a multiple of the batch stride (SV_STREAM_UNROLL * 2048 logits),
  // so only a row's last chunk has a partial batch.
  L.chunk = kChunk;
  L.nc = (int)(((int64_t)V + L.chunk - 1) / L.chunk);
  L.ntile = (V + kTile - 1) / kTile;
  L.nt = (L.ntile + kTilesPerItem - 1) / kTilesPerItem;
  const size_t R = 2 * (size_t)gamma + 1;
  size_t off = 0;
  L.err_off = off;
  off += 256;
  L.part_off = off;
  off += align256((size_t)B * R * L.nc * sizeof(uint64_t));
  L.mraw_off = off;
  off += align256((size_t)B * R * L.nc * sizeof(unsigned));
  L.seq_off = off;
  off += align256((size_t)B * sizeof(SeqRec));
  L.flag_off = off;
  off += align256((size_t)B * kFlagStride * sizeof(unsigned));
  L.tiles_off = off;
  off += align256((size_t)B * L.ntile * sizeof(uint64_t));
  L.mass_off = off;
  off += align256((size_t)B * L.nt * sizeof(uint64_t));
  L.rsum_off = off;
  off += align256((size_t)B * L.nt * sizeof(uint64_t));
  L.cpart_off = off;
  off += align256((size_t)B * (gamma + 1) * L.nc * sizeof(Top3));
  L.topp_off = off;
  off += align256((size_t)B * R * sizeof(TopPRow));
  L.hist_off = off;
  off += align256((size_t)B * R * kDigits * sizeof(double));
  L.total = B == 0 ? 0 : off;
  return L;
}

// Work-groups of the fused kernel the device holds at once (cached per device).
template <int DT, bool VEC, bool PRED, bool EARLY>
static hipError_t resident_groups(int& slots) {
  static int cache[64][2][2][2][2];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int* c = dev >= 0 && dev < 64 ? &cache[dev][DT][VEC ? 1 : 0][PRED ? 1 : 0][EARLY ? 1 : 0] : nullptr;
  if (c && *c > 0) {
    slots = *c;
    return hipSuccess;
  }
  int ncu = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(fused_kernel<DT, VEC, SV_STREAM_UNROLL, PRED, EARLY>),
        kThreads, 0);
  if (e != hipSuccess) return e;
  slots = std::max(1, ncu * per_cu);
  if (c) *c = slots;
  return hipSuccess;
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

template <int DT, bool VEC>
static hipError_t launch_kernels(const VerifyArgs& a, hipStream_t st);

// pa: NULL, or outcome prediction after the verification.
template <int DT, bool VEC>
static hipError_t launch_all(const VerifyArgs& a, const PredictArgs* pa, hipStream_t st) {
  // The single-kernel order for packed bf16 rows; float32 or unaligned rows
  // take one kernel per item kind (their sampling paths need more registers
  // than the stream items' occupancy leaves) and the stand-alone prediction.
  if constexpr (SV_FUSED && DT == kBF16 && VEC) {
    if (!a.topp && !(a.saguaro && a.eps > 0.f)) {
      int slots = 0;
      const bool eps_mode = a.saguaro && a.eps > 0.f;
      if (a.early) {
        hipError_t e = resident_groups<DT, VEC, false, true>(slots);
        if (e != hipSuccess) return e;
        static_assert(SV_EARLY_CHUNK % SV_CHUNK == 0, "early-exit chunks are whole default chunks");
        VerifyArgs b = a;   // never more chunks than the workspace holds
        b.chunk = SV_EARLY_CHUNK;
        b.nc = (int)(((int64_t)a.V + b.chunk - 1) / b.chunk);
        const Sched sc = make_sched_early(b.B, b.gamma, b.nc, eps_mode ? b.nt : 0, b.nt, slots);
        hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, false, true>), dim3((unsigned)sc.total),
                           dim3(kThreads), 0, st, b, sc);
        return hipGetLastError();
      }
      hipError_t e = pa ? resident_groups<DT, VEC, true, false>(slots) : resident_groups<DT, VEC, false, false>(slots);
      if (e != hipSuccess) return e;
      const Sched sc = make_sched(a.B, 2 * a.gamma * a.nc, (pa ? 2 : 1) * a.nc, eps_mode ? a.nt : 0, a.nt, slots);
      if (pa) {
        hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, true, false>), dim3((unsigned)sc.total),
                           dim3(kThreads), 0, st, a, sc);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return predict_launch_leaders(*pa, SPEC_BF16, st);
      }
      hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, false, false>), dim3((unsigned)sc.total),
                         dim3(kThreads), 0, st, a, sc);
      return hipGetLastError();
    }
  }
  {
    hipError_t e = launch_kernels<DT, VEC>(a, st);
    if (e != hipSuccess || !pa) return e;
    return predict_launch_rows(*pa, DT == kBF16 ? SPEC_BF16 : SPEC_F32, VEC, st);
  }
}

template <int DT, bool VEC, bool CUT>
static hipError_t launch_kernels_cut(const VerifyArgs& a, hipStream_t st) {
  const int R = 2 * a.gamma + 1;
  const bool eps_mode = a.saguaro && a.eps > 0.f;
  const unsigned nstream = (unsigned)((int64_t)a.B * R * a.nc);
  const unsigned nsample = (unsigned)((int64_t)a.B * a.nt);
  const unsigned rows = (unsigned)((int64_t)a.B * R);
  if (CUT && DT == kBF16 && a.V <= kCountMaxV) {
    // Counting gives each row's nucleus and its normaliser piece in one read.
    int ncu = 0, dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((topp_count_kernel<VEC>), dim3(std::min<unsigned>(rows, (unsigned)std::max(ncu, 1))),
                       dim3(kCountThreads), 0, st, a, (int64_t)rows);
  } else {
    hipLaunchKernelGGL((stream_kernel<DT, VEC, SV_STREAM_UNROLL>), dim3(nstream), dim3(kThreads), 0, st, a);
    if constexpr (CUT) {   // the nucleus of every row by radix selection
      constexpr int npass = DT == kBF16 ? 2 : 4;
      hipLaunchKernelGGL(topp_init_kernel, dim3(rows), dim3(64), 0, st, a);
      for (int pass = 0; pass < npass; ++pass) {
        hipLaunchKernelGGL((topp_hist_kernel<DT, VEC>), dim3(nstream), dim3(kThreads), 0, st, a, pass);
        hipLaunchKernelGGL((topp_select_kernel<DT>), dim3(rows), dim3(64), 0, st, a, pass, npass);
      }
    }
  }
  if (a.early)   // position-major: the test of (i - 1, b) has a smaller block number than (i, b)'s
    hipLaunchKernelGGL((test_kernel<DT>), dim3((unsigned)((int64_t)a.gamma * a.B)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decide_kernel<DT, CUT>), dim3((unsigned)a.B), dim3(kThreads), 0, st, a);
  if (eps_mode) hipLaunchKernelGGL((mass_kernel<DT, VEC, CUT>), dim3(nsample), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((sample_kernel<DT, VEC, CUT>), dim3(nsample), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((draw_kernel<DT, VEC, CUT>), dim3((unsigned)a.B), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((final_kernel<DT>), dim3((unsigned)a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int DT, bool VEC>
static hipError_t launch_kernels(const VerifyArgs& a, hipStream_t st) {
  return a.topp ? launch_kernels_cut<DT, VEC, true>(a, st) : launch_kernels_cut<DT, VEC, false>(a, st);
}

static int verify_impl(const void* draft, const void* target, int dtype, const int32_t* tokens,
                       const float* u_acc, const float* u_smp, int B, int gamma, int V, float T,
                       const int32_t* in_len, int32_t* out_tokens, int32_t* out_acc,
                       int32_t* out_fr, uint64_t* out_mask, int32_t* out_len,
                       const spec_diag* diag, void* ws, size_t ws_bytes, void* stream,
                       int saguaro, float eps, int32_t* cand = nullptr, int32_t* hit = nullptr,
                       int32_t* cand_idx = nullptr, int early = 0, const float* temps = nullptr,
                       float top_p = 1.f) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (!sizes_ok(B, gamma, V)) return SPEC_EINVAL;
  if (!temps && (!(T > 0.f) || !std::isfinite(T))) return SPEC_EINVAL;
  if (temps) T = 1.f;   // unused: every sequence has its own
  if (!(eps >= 0.f) || !std::isfinite(eps)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!draft || !target || !tokens || !u_acc || !u_smp || !out_tokens || !out_acc)
    return SPEC_EINVAL;
  const Layout L = layout(B, gamma, V);
  // Every launch (and the fused kernel's item count) stays within one grid
  // dimension of 2^32 - 1 work-items, with block numbers below 2^31.
  const int64_t items = (int64_t)B * ((2 * gamma + 2) * L.nc + 2 * L.nt + 3 + gamma);
  if (items * kThreads > (int64_t)UINT_MAX || items > (int64_t)INT_MAX) return SPEC_EINVAL;
  if (!ws || ws_bytes < L.total) return SPEC_EWORKSPACE;

  VerifyArgs a;
  a.draft = draft;
  a.target = target;
  a.tokens = tokens;
  a.u_acc = u_acc;
  a.u_smp = u_smp;
  a.in_len = in_len;
  a.out_tokens = out_tokens;
  a.out_acc = out_acc;
  a.out_first_reject = out_fr;
  a.out_mask = out_mask;
  a.out_len = out_len;
  if (diag) a.diag = *diag;
  else a.diag = spec_diag{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  char* w = static_cast<char*>(ws);
  a.err = reinterpret_cast<unsigned*>(w + L.err_off);
  a.part = reinterpret_cast<uint64_t*>(w + L.part_off);
  a.mraw = reinterpret_cast<unsigned*>(w + L.mraw_off);
  a.seq = reinterpret_cast<SeqRec*>(w + L.seq_off);
  a.flag = reinterpret_cast<unsigned*>(w + L.flag_off);
  a.tiles = reinterpret_cast<uint64_t*>(w + L.tiles_off);
  a.mass = reinterpret_cast<uint64_t*>(w + L.mass_off);
  a.rsum = reinterpret_cast<uint64_t*>(w + L.rsum_off);
  a.cpart = reinterpret_cast<Top3*>(w + L.cpart_off);
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.nc = L.nc;
  a.chunk = L.chunk;
  a.ntile = L.ntile;
  a.nt = L.nt;
  {
    // c_hi is rounded toward zero so that c_lo > 0: a -inf logit then gives
    // fma(-inf, c_lo, -inf) = -inf, never NaN.
    const double c = 1.4426950408889634073599246810019 / (double)T;
    float ch = (float)c;
    if ((double)ch >= c) ch = std::nextafter(ch, 0.f);
    a.c_hi = ch;
    a.c_lo = (float)(c - (double)ch);
    if (!(a.c_lo > 0.f)) a.c_lo = 1.17549435e-38f;
    a.cTd = (double)a.c_hi + (double)a.c_lo;
    a.invT = 1.0 / (double)T;
  }
  a.saguaro = saguaro;
  a.eps = eps;
  a.early = early;
  a.temps = temps;
  a.top_p = top_p;
  a.topp = nullptr;
  a.hist = nullptr;
  if (top_p < 1.f) {
    a.topp = reinterpret_cast<TopPRow*>(w + L.topp_off);
    a.hist = reinterpret_cast<double*>(w + L.hist_off);
  }

  PredictArgs p;
  if (cand) {
    p.draft = draft;
    p.accepted = out_acc;
    p.out_tokens = out_tokens;
    p.cand = cand;
    p.hit = hit;
    p.cand_idx = cand_idx;
    p.part = a.cpart;
    p.B = B;
    p.gamma = gamma;
    p.V = V;
    p.nc = L.nc;
    p.chunk = L.chunk;
  }
  const PredictArgs* pa = cand ? &p : nullptr;
  const bool vec = (V % 8 == 0) && ((uintptr_t)draft % 16 == 0) && ((uintptr_t)target % 16 == 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e;
  if (dtype == SPEC_BF16) e = vec ? launch_all<kBF16, true>(a, pa, st) : launch_all<kBF16, false>(a, pa, st);
  else e = vec ? launch_all<kF32, true>(a, pa, st) : launch_all<kF32, false>(a, pa, st);
  return e == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

}  // namespace sv

extern "C" {

size_t spec_workspace_bytes(int B, int gamma, int V, int dtype) {
  if ((dtype != SPEC_F32 && dtype != SPEC_BF16) || !sv::sizes_ok(B, gamma, V)) return 0;
  return sv::layout(B, gamma, V).total;
}

int spec_verify(const void* draft_logits, const void* target_logits, int dtype,
                const int32_t* draft_tokens, const float* u_accept, const float* u_sample, int B,
                int gamma, int V, float temperature, const int32_t* in_len, int32_t* out_tokens,
                int32_t* out_accepted, int32_t* out_first_reject, uint64_t* out_accept_mask,
                int32_t* out_len, const spec_diag* diag, void* workspace, size_t workspace_bytes,
                void* stream) {
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, 0, 0.f);
}

int spec_verify_saguaro(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        int B, int gamma, int V, float temperature, const int32_t* in_len,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                        uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                        void* workspace, size_t workspace_bytes, void* stream, float eps) {
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, 1, eps);
}

int spec_verify_predict(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        int B, int gamma, int V, float temperature, const int32_t* in_len,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                        uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                        int saguaro, float eps, int32_t* cand, int32_t* hit, int32_t* cand_idx,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!cand || (saguaro != 0 && saguaro != 1)) return SPEC_EINVAL;
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, saguaro,
                         eps, cand, hit, cand_idx);
}

int spec_verify_early(const void* draft_logits, const void* target_logits, int dtype,
                      const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                      int B, int gamma, int V, float temperature, const int32_t* in_len,
                      int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                      uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                      int saguaro, float eps, void* workspace, size_t workspace_bytes, void* stream) {
  if (saguaro != 0 && saguaro != 1) return SPEC_EINVAL;
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, saguaro,
                         eps, nullptr, nullptr, nullptr, 1);
}

int spec_verify_ex(const void* draft_logits, const void* target_logits, int dtype,
                   const int32_t* draft_tokens, const float* u_accept, const float* u_sample, int B,
                   int gamma, int V, float temperature, const int32_t* in_len, int32_t* out_tokens,
                   int32_t* out_accepted, int32_t* out_first_reject, uint64_t* out_accept_mask,
                   int32_t* out_len, const spec_diag* diag, const spec_options* opts,
                   void* workspace, size_t workspace_bytes, void* stream) {
  spec_options o{};
  if (opts) o = *opts;
  if (o.saguaro != 0 && o.saguaro != 1) return SPEC_EINVAL;
  if (o.early && o.cand) return SPEC_EINVAL;
  if (!(o.top_p >= 0.f && o.top_p <= 1.f)) return SPEC_EINVAL;   // NaN included
  const float top_p = o.top_p > 0.f ? o.top_p : 1.f;
  if (o.early && top_p < 1.f) return SPEC_EINVAL;
  if (!o.cand && (o.hit || o.cand_idx)) return SPEC_EINVAL;
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream,
                         o.saguaro, o.saguaro ? o.eps : 0.f, o.cand, o.hit, o.cand_idx, o.early ? 1 : 0,
                         o.temperature, top_p);
}

const char* spec_status_str(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument (size, temperature, eps or NULL pointer)";
    case SPEC_EDTYPE: return "unknown dtype (expected SPEC_F32 or SPEC_BF16)";
    case SPEC_EWORKSPACE: return "workspace missing or smaller than spec_workspace_bytes()";
    case SPEC_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
