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
//   stream item (b, r, c): stream chunk c of row r of sequence b once from
//     HBM and reduce it to a piece of the tempered-softmax normaliser,
//     (mc, s) with s = sum_j 2^(l_j * c_T - mc), c_T = log2(e) / T.  c_T is
//     an unevaluated float pair (two FMAs per logit) so the temperature is
//     exact; mc is an integer, so rescaling a sum is an exact ldexp.  Each
//     batch of a lane's logits is tree-summed in fp32 and accumulated in fp64.
//     The last item of a sequence to finish (arrival counter) merges the
//     pieces in fp64, runs the accept test at every draft position (fp64,
//     wave ballot -> first rejection k) and writes the sequence's decision.
//   sample item (b, s): per-tile (2048-logit) sums of the sampling weights
//     over its tiles of row pair k (or target row gamma).  The last item of a
//     sequence locates the tile holding u * total (fp64 scan over the tile
//     sums), rescans that tile (fp64 prefix over the same per-lane fp32 sums)
//     and writes the outputs.  Saguaro with eps > 0 runs one more set of
//     items first to get the residual mass the clamp is relative to.
//
// Workspace counters are zero between calls; the last arriver of each phase
// resets its counter.
#include "common.h"
#include "spec_verify.h"

#include <cmath>
#include <limits.h>
#include <algorithm>
#include <type_traits>

namespace sv {

// One (row, chunk) piece of a row's normaliser: s = sum 2^(l*c_T - mc), mc an
// integer (log2 units); mraw = the chunk's largest raw logit.
struct Partial {
  float mc;
  float mraw;
  double s;
};

__device__ __forceinline__ void store_partial(Partial* p, float mc, float mraw, double s) {
  const uint64_t w = (uint64_t)__float_as_uint(mc) | ((uint64_t)__float_as_uint(mraw) << 32);
  st_dev_u64(reinterpret_cast<uint64_t*>(p), w);
  st_dev(&p->s, s);
}

__device__ __forceinline__ Partial load_partial(const Partial* p) {
  const uint64_t w = ld_dev_u64(reinterpret_cast<const uint64_t*>(p));
  Partial r;
  r.mc = __uint_as_float((uint32_t)w);
  r.mraw = __uint_as_float((uint32_t)(w >> 32));
  r.s = ld_dev(&p->s);
  return r;
}

enum : int { kModeTarget = 0, kModeResidual = 1, kModeSaguaro = 2, kModeSaguaroEps = 3 };

#ifndef SV_TILES_PER_ITEM
#define SV_TILES_PER_ITEM 4
#endif
#ifndef SV_STREAM_UNROLL
#define SV_STREAM_UNROLL 4
#endif
// 1: one persistent cooperative kernel runs every phase (the default);
// 0: separate stream, decision and sampling kernels.
#ifndef SV_FUSED
#define SV_FUSED 0
#endif
// Sampling items of a sequence run this many rounds of the persistent grid
// after its stream items (x1000).
// Waves per SIMD the fused kernel is compiled for (registers are capped to
// fit; the rare decision and refine paths may spill).
#ifndef SV_FUSED_WAVES
#define SV_FUSED_WAVES 8
#endif
#ifndef SV_LAG_MILLIROUNDS
#define SV_LAG_MILLIROUNDS 1500
#endif
constexpr int kTilesPerItem = SV_TILES_PER_ITEM;
static_assert(kChunk % (SV_STREAM_UNROLL * kThreads * kUnit) == 0,
              "a stream chunk must hold whole batches");

// A sequence's decision, written by its last stream item.
struct SeqRec {
  uint64_t mask;
  int k;
  int valid;
  int mode;         // weights of the draw
  float Mt;         // offset of the row drawn from (target row k)
  float K_hi, K_lo; // log2(p_j/q_j) = (ld_j - lt_j) * c_T + K
  float epsS;       // eps * sum of residual weights (Saguaro eps > 0)
  float pad0;
  double Zt;        // normaliser of target row k (offset Mt)
  double pad1;
};

static_assert(sizeof(SeqRec) % 8 == 0, "SeqRec is moved as 64-bit words");
constexpr int kRecWords = sizeof(SeqRec) / 8;

// A decision record written and read with device-coherent 64-bit accesses.
__device__ __forceinline__ void store_rec(SeqRec* p, const SeqRec& r) {
  const uint64_t* w = reinterpret_cast<const uint64_t*>(&r);
#pragma unroll
  for (int i = 0; i < kRecWords; ++i) st_dev_u64(reinterpret_cast<uint64_t*>(p) + i, w[i]);
}
__device__ __forceinline__ SeqRec load_rec(const SeqRec* p) {
  SeqRec r;
  uint64_t* w = reinterpret_cast<uint64_t*>(&r);
#pragma unroll
  for (int i = 0; i < kRecWords; ++i) w[i] = ld_dev_u64(reinterpret_cast<const uint64_t*>(p) + i);
  return r;
}
// epsS and pad0 share the fifth word.
__device__ __forceinline__ void store_rec_eps(SeqRec* p, float epsS) {
  st_dev_u64(reinterpret_cast<uint64_t*>(p) + 4, (uint64_t)__float_as_uint(epsS));
}

// Arrival counters and ready flags of one sequence, one 128-byte line each.
struct SeqCtr {
  unsigned stream_done;  // stream items finished
  unsigned a_done;       // residual-mass items finished (Saguaro eps > 0)
  unsigned b_done;       // sampling items finished
  unsigned decided;      // 1 once the decision record is written
  unsigned a_ready;      // 1 once eps * residual mass is written
  unsigned pad[27];
};

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
  unsigned* err;     // nonzero if a bounded wait timed out (co-residency lost)
  unsigned* next;    // item counter of the fused kernel (zero between calls)
  Partial* part;     // [B][2*gamma+1][nc]
  SeqRec* seq;       // [B]
  SeqCtr* ctr;       // [B]
  double* tiles;     // [B][ntile] tile sums of the sampling weights
  double* itemsum;   // [B][nt] residual-weight sum of each sample item
  int B, gamma, V;
  int nc, chunk;     // stream chunks per row and their length
  int ntile, nt;     // sampling tiles per row; sample items per sequence
  float c_hi, c_lo;  // log2(e) / T as an unevaluated float pair, c_lo > 0
  double cTd;        // c_hi + c_lo
  double invT;
  int saguaro;
  float eps;
};

template <int DT>
__device__ __forceinline__ const void* row_ptr(const VerifyArgs& a, int b, int r) {
  // r < gamma: draft row r; otherwise target row r - gamma.
  const int64_t es = DT == kBF16 ? 2 : 4;
  const bool is_draft = r < a.gamma;
  const int64_t idx = (int64_t)b * (a.gamma + 1) + (is_draft ? r : r - a.gamma);
  const char* base = static_cast<const char*>(is_draft ? a.draft : a.target);
  return base + idx * a.V * es;
}

// Thread 0 (which wrote this work-group's payload with device-coherent
// stores) waits for them to complete and counts the arrival.  Returns true in
// every thread of the work-group that completes the count; that work-group
// reads the other arrivers' payloads with device-coherent loads.
__device__ __forceinline__ bool arrive(unsigned* counter, unsigned total, int* lds_flag) {
  __syncthreads();
  if (threadIdx.x == 0) {
    wait_mem();
    const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = (old == total - 1);
    if (last)   // nobody else touches it again in this call
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = last;
  }
  __syncthreads();
  return *lds_flag != 0;
}

// ---------------------------------------------------------------------------
// Stream item: one chunk of one row -> Partial.

// One batch of N units (8 logits each) of a lane: raise the lane's integer
// offset if the batch holds a larger logit (rescaling the running sum by an
// exact power of two), then add the batch's terms 2^(l c_T - mref), tree-summed
// in fp32, to the fp64 running sum.
template <int DT, bool VEC, int N>
__device__ __forceinline__ void stream_batch(const Raw8<DT, VEC> (&raw)[N], float ch, float cl,
                                             float& mref, float& mraw, double& s) {
  float v[N * 8];
#pragma unroll
  for (int u = 0; u < N; ++u) unpack<DT, VEC>(raw[u], *reinterpret_cast<float(*)[8]>(v + u * 8));
  float bm = v[0];
#pragma unroll
  for (int e = 1; e < N * 8; ++e) bm = fmaxf(bm, v[e]);
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

template <int DT, bool VEC, int U>
__device__ __forceinline__ void stream_item(const VerifyArgs& a, int b, int r, int c, float* lds_f,
                                            double* lds_d) {
  const void* row = row_ptr<DT>(a, b, r);
  const int64_t begin = (int64_t)c * a.chunk;
  const int64_t end = min<int64_t>(begin + a.chunk, a.V);
  const float ch = a.c_hi, cl = a.c_lo;

  // mref: this lane's integer offset (log2 units); s: fp64 sum of 2^(l*c_T - mref).
  float mref = kNegSentinel, mraw = -INFINITY;
  double s = 0.0;
  constexpr int64_t kStep = (int64_t)kThreads * kUnit;
  int64_t j = begin + (int64_t)threadIdx.x * kUnit;
  // Full batches: U units, all in range, loads issued back to back.
  for (; j + (U - 1) * kStep + kUnit <= end; j += U * kStep) {
    Raw8<DT, VEC> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load_raw<DT, VEC>(row, j + u * kStep, end, raw[u]);
    stream_batch<DT, VEC, U>(raw, ch, cl, mref, mraw, s);
  }
  // Remaining units of this lane (fewer than U; the last may be partial).
  for (; j < end; j += kStep) {
    Raw8<DT, VEC> raw[1];
    load_raw<DT, VEC>(row, j, end, raw[0]);
    stream_batch<DT, VEC, 1>(raw, ch, cl, mref, mraw, s);
  }
  // Merge the lanes: wave shuffles, then one barrier; thread 0 stores the piece.
  const float wm = wave_max(mref);
  const float wr = wave_max(mraw);
  double sd = (s != 0.0) ? ldexp(s, (int)fmaxf(mref - wm, -2000.f)) : 0.0;
  sd = wave_sum(sd);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    lds_f[wave] = wm;
    lds_f[kWaves + wave] = wr;
    lds_d[wave] = sd;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mb = lds_f[0], mr = lds_f[kWaves];
    for (int i = 1; i < kWaves; ++i) {
      mb = fmaxf(mb, lds_f[i]);
      mr = fmaxf(mr, lds_f[kWaves + i]);
    }
    double sb = 0.0;
    for (int i = 0; i < kWaves; ++i)
      if (lds_d[i] != 0.0) sb += ldexp(lds_d[i], (int)fmaxf(lds_f[i] - mb, -2000.f));
    store_partial(a.part + ((int64_t)b * (2 * a.gamma + 1) + r) * a.nc + c, mb, mr, sb);
  }
}

// ---------------------------------------------------------------------------
// Decision of one sequence.

struct DecideLds {
  float M[128];
  double Z[128];
  int bad[128];
  uint64_t mask;
  int k, valid;
};

// Merge the chunk pieces of every row (16 lanes per row, 16 rows per pass;
// fp64), then run the accept test at every draft position (wave 0, lane i =
// position i; fp64) and record the sequence's decision.
template <int DT>
__device__ void decide_seq(const VerifyArgs& a, int b, DecideLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = a.gamma, R = 2 * g + 1;
  const double cTd = a.cTd;
  const Partial* P0 = a.part + (int64_t)b * R * a.nc;
  const int sub = lane & 15;
  for (int r0 = 0; r0 < R; r0 += 16) {
    const int r = r0 + wave * 4 + (lane >> 4);
    float M = kNegSentinel, mr = -INFINITY;
    double z = 0.0;
    if (r < R) {
      const Partial* P = P0 + (int64_t)r * a.nc;
      if (a.nc <= 16) {   // one piece per lane, kept in registers
        const Partial p = sub < a.nc ? load_partial(P + sub) : Partial{kNegSentinel, -INFINITY, 0.0};
        M = p.mc;
        mr = p.mraw;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
          M = fmaxf(M, __shfl_xor(M, o, 16));
          mr = fmaxf(mr, __shfl_xor(mr, o, 16));
        }
        if (p.s != 0.0) z = ldexp(p.s, (int)fmaxf(p.mc - M, -2000.f));
      } else {
        for (int c = sub; c < a.nc; c += 16) {
          const Partial p = load_partial(P + c);
          M = fmaxf(M, p.mc);
          mr = fmaxf(mr, p.mraw);
        }
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
          M = fmaxf(M, __shfl_xor(M, o, 16));
          mr = fmaxf(mr, __shfl_xor(mr, o, 16));
        }
        for (int c = sub; c < a.nc; c += 16) {
          const Partial p = load_partial(P + c);
          if (p.s != 0.0) z += ldexp(p.s, (int)fmaxf(p.mc - M, -2000.f));
        }
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) z += __shfl_xor(z, o, 16);
    if (r < R && sub == 0) {
      const int ok = (z > 0.0) && isfinite(z) && isfinite(M);
      sh.M[r] = M;
      sh.Z[r] = z;
      sh.bad[r] = !ok;
      if (ok && a.diag.row_max) a.diag.row_max[(int64_t)b * R + r] = (double)mr * a.invT;
      if (ok && a.diag.row_logZ)
        a.diag.row_logZ[(int64_t)b * R + r] = (double)M * 0.69314718055994530942 + log(z);
    }
  }
  __syncthreads();

  if (wave == 0) {
    int rows_bad = 0;
    for (int r = lane; r < R; r += 64) rows_bad |= sh.bad[r];
    rows_bad = __ballot(rows_bad) != 0;
    int acc = 0, bad = 0;
    if (lane < g) {
      const int x = a.tokens[(int64_t)b * g + lane];
      bad = (x < 0 || x >= a.V);
      if (!bad && !rows_bad) {
        const float ld = load_one<DT>(row_ptr<DT>(a, b, lane), x);
        const float lt = load_one<DT>(row_ptr<DT>(a, b, g + lane), x);
        const double px = exp2((double)ld * cTd - (double)sh.M[lane]) / sh.Z[lane];
        const double qx = exp2((double)lt * cTd - (double)sh.M[g + lane]) / sh.Z[g + lane];
        double ratio;
        if (px > 0.0) ratio = fmin(1.0, qx / px);
        else ratio = qx > 0.0 ? 1.0 : 0.0;
        acc = (double)a.u_acc[(int64_t)b * g + lane] < ratio;
        if (a.diag.px) a.diag.px[(int64_t)b * g + lane] = px;
        if (a.diag.qx) a.diag.qx[(int64_t)b * g + lane] = qx;
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
  const int64_t orow = (int64_t)b * (g + 1);
  if (!sh.valid) {
    if (tid <= g) a.out_tokens[orow + tid] = -1;
    if (tid == 0) {
      a.out_acc[b] = -1;
      if (a.out_first_reject) a.out_first_reject[b] = -1;
      if (a.out_mask) a.out_mask[b] = 0;
      if (a.out_len) a.out_len[b] = a.in_len ? a.in_len[b] : 0;
    }
  }
  if (tid == 0) {
    SeqRec rec;
    rec.mask = sh.mask;
    rec.k = k;
    rec.valid = sh.valid;
    rec.mode = k == g ? kModeTarget
                      : (!a.saguaro ? kModeResidual : (a.eps > 0.f ? kModeSaguaroEps : kModeSaguaro));
    rec.Mt = sh.M[g + k];
    const double K = k < g ? ((double)sh.M[g + k] - (double)sh.M[k]) + log2(sh.Z[g + k] / sh.Z[k]) : 0.0;
    rec.K_hi = (float)K;
    rec.K_lo = (float)(K - (double)rec.K_hi);
    rec.epsS = 0.f;
    rec.pad0 = 0.f;
    rec.Zt = sh.Z[g + k];
    rec.pad1 = 0.0;
    store_rec(a.seq + b, rec);
  }
}

// ---------------------------------------------------------------------------
// Sampling weights.

struct SampleCoef {
  float c_hi, c_lo, Mt, K_hi, K_lo, epsS;
};

__device__ __forceinline__ SampleCoef coef_of(const VerifyArgs& a, const SeqRec& rec) {
  SampleCoef c;
  c.c_hi = a.c_hi;
  c.c_lo = a.c_lo;
  c.Mt = rec.Mt;
  c.K_hi = rec.K_hi;
  c.K_lo = rec.K_lo;
  c.epsS = rec.epsS;
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
  } else {
    const float dl = ld - lt;
    float d;
    if constexpr (DT == kBF16) {
      d = fmaf(dl, c.c_hi, c.K_hi) + fmaf(dl, c.c_lo, c.K_lo);   // dl is exact
    } else {
      const float bb = dl - ld;
      const float err = (ld - (dl - bb)) - (lt + bb);             // ld - lt = dl + err
      d = fmaf(dl, c.c_hi, c.K_hi) + fmaf(err, c.c_hi, fmaf(dl, c.c_lo, c.K_lo));
    }
    const float ex = exp2_fast(d);          // p_j / q_j
    const float em1 = one_minus_exp2<PRECISE>(d, ex);
    const bool pos = (eq > 0.f) && (d < 0.f);
    const float res = pos ? eq * em1 : 0.f;
    r = res;
    if constexpr (MODE == kModeResidual) return res;
    else if constexpr (MODE == kModeSaguaro) return pos ? eq * sqrtf(ex * em1) : 0.f;
    else return (eq > 0.f) ? sqrtf(eq * ex * fmaxf(res, c.epsS)) : 0.f;
  }
}

template <int DT, int MODE, bool PRECISE>
__device__ __forceinline__ void sample_weights(const float (&ld)[8], const float (&lt)[8],
                                               const SampleCoef& c, float (&w)[8], float (&r)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = weight_one<DT, MODE, PRECISE>(ld[e], lt[e], c, r[e]);
}

// Mode chosen at run time (scalar paths: pi(y), degenerate fallbacks).
template <int DT, bool PRECISE>
__device__ __noinline__ float weight_rt(int mode, float ld, float lt, const SampleCoef& c, float& r) {
  switch (mode) {
    case kModeTarget: return weight_one<DT, kModeTarget, PRECISE>(ld, lt, c, r);
    case kModeResidual: return weight_one<DT, kModeResidual, PRECISE>(ld, lt, c, r);
    case kModeSaguaro: return weight_one<DT, kModeSaguaro, PRECISE>(ld, lt, c, r);
    default: return weight_one<DT, kModeSaguaroEps, PRECISE>(ld, lt, c, r);
  }
}

// Call f with the weight mode as a compile-time constant.
template <class F>
__device__ __forceinline__ void with_mode(int mode, F&& f) {
  switch (mode) {
    case kModeTarget: f(std::integral_constant<int, kModeTarget>{}); break;
    case kModeResidual: f(std::integral_constant<int, kModeResidual>{}); break;
    case kModeSaguaro: f(std::integral_constant<int, kModeSaguaro>{}); break;
    default: f(std::integral_constant<int, kModeSaguaroEps>{}); break;
  }
}

template <int DT, bool VEC, int MODE>
__device__ __forceinline__ void load_pair(const void* drow, const void* trow, int64_t j0, int64_t V,
                                          float (&ld)[8], float (&lt)[8]) {
  if (j0 < V) {
    load8<DT, VEC>(trow, j0, V, lt);
    if constexpr (MODE != kModeTarget) load8<DT, VEC>(drow, j0, V, ld);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) lt[e] = ld[e] = -INFINITY;
  }
}

// Rows of the draw: target row k and (on a rejection) draft row k.
template <int DT>
__device__ __forceinline__ void draw_rows(const VerifyArgs& a, int b, int k, const void*& drow,
                                          const void*& trow) {
  drow = row_ptr<DT>(a, b, k < a.gamma ? k : 0);
  trow = row_ptr<DT>(a, b, a.gamma + k);
}

// Tile sums of the weights over tiles [t0, t0 + kTilesPerItem) (clipped to
// ntile): tw[i] (fp64, identical in every thread) and, last, the residual total.
template <int DT, bool VEC, int MODE>
__device__ __forceinline__ void tile_sums(const VerifyArgs& a, int b, const SampleCoef& cf, int k,
                                          int t0, double (&tw)[kTilesPerItem + 1], double* lds_d) {
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  const int64_t lane_off = (int64_t)threadIdx.x * kUnit;
  Raw8<DT, VEC> rd[kTilesPerItem], rt[kTilesPerItem];
#pragma unroll
  for (int i = 0; i < kTilesPerItem; ++i) {
    const int t = t0 + i;
    const int64_t j0 = t < a.ntile ? (int64_t)t * kTile + lane_off : (int64_t)a.V;
    load_raw<DT, VEC>(trow, j0, a.V, rt[i]);
    if constexpr (MODE != kModeTarget) load_raw<DT, VEC>(drow, j0, a.V, rd[i]);
  }
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < kTilesPerItem; ++i) {
    float ld[8], lt[8], w[8], r[8];
    unpack<DT, VEC>(rt[i], lt);
    if constexpr (MODE != kModeTarget) unpack<DT, VEC>(rd[i], ld);
    sample_weights<DT, MODE, false>(ld, lt, cf, w, r);
    float ws = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ws += w[e];
      rs += r[e];
    }
    tw[i] = (double)ws;
  }
  tw[kTilesPerItem] = (double)rs;
  block_sum_n<kTilesPerItem + 1>(tw, lds_d);
}

// ---------------------------------------------------------------------------
// Sample items.

// Residual mass for the Saguaro clamp (pass A).
template <int DT, bool VEC>
__device__ void sample_item_a(const VerifyArgs& a, int b, int s, double* lds_d) {
  const SeqRec rec = load_rec(a.seq + b);
  double tw[kTilesPerItem + 1] = {};
  if (rec.valid && rec.mode == kModeSaguaroEps)
    tile_sums<DT, VEC, kModeResidual>(a, b, coef_of(a, rec), rec.k, s * kTilesPerItem, tw, lds_d);
  if (threadIdx.x == 0) st_dev(a.itemsum + (int64_t)b * a.nt + s, tw[kTilesPerItem]);
}

// eps * residual mass, by the last pass-A item of a sequence.
__device__ void finish_a(const VerifyArgs& a, int b, double* lds_d) {
  double v = 0.0;
  for (int i = threadIdx.x; i < a.nt; i += kThreads) v += ld_dev(a.itemsum + (int64_t)b * a.nt + i);
  v = block_sum(v, lds_d);
  if (threadIdx.x == 0) store_rec_eps(a.seq + b, (float)(v * (double)a.eps));
}

// Tile sums of the sampling weights (pass B).
template <int DT, bool VEC>
__device__ void sample_item_b(const VerifyArgs& a, int b, int s, double* lds_d) {
  const SeqRec rec = load_rec(a.seq + b);
  if (!rec.valid) return;
  const int t0 = s * kTilesPerItem;
  const SampleCoef cf = coef_of(a, rec);
  with_mode(rec.mode, [&](auto m) {
    double tw[kTilesPerItem + 1];
    tile_sums<DT, VEC, decltype(m)::value>(a, b, cf, rec.k, t0, tw, lds_d);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int i = 0; i < kTilesPerItem; ++i)
        if (t0 + i < a.ntile) st_dev(a.tiles + (int64_t)b * a.ntile + t0 + i, tw[i]);
      st_dev(a.itemsum + (int64_t)b * a.nt + s, tw[kTilesPerItem]);
    }
  });
}

struct RefineLds {
  double lds_d[kWaves * (kTilesPerItem + 1)];
  int lds_i[kWaves];
  int tile;
  double off, lo, hi, w;
};

// Locate the tile holding u * S (S = sum of the tile sums) by an fp64 scan
// over the tile sums in token order; returns S, sets sh.tile and sh.off.
__device__ double locate_tile(const double* tiles, int ntile, double u, RefineLds& sh, double& target) {
  const int tid = threadIdx.x;
  double S = 0.0;
  if (ntile <= kThreads) {   // one tile sum per thread, loaded once
    const double v = tid < ntile ? ld_dev(tiles + tid) : 0.0;
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
    for (int i = tid; i < ntile; i += kThreads) v += ld_dev(tiles + i);
    S = block_sum(v, sh.lds_d);
    target = u * S;
    double carry = 0.0;
    for (int base = 0; base < ntile; base += kThreads) {
      const int t = base + tid;
      const double x = t < ntile ? ld_dev(tiles + t) : 0.0;
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
      if (ld_dev(tiles + t) > 0.0) last = t;
    last = -block_min_int(-last, sh.lds_i);
    if (tid == 0) {
      sh.tile = max(last, 0);
      double off = 0.0;
      for (int t = 0; t < last; ++t) off += ld_dev(tiles + t);
      sh.off = off;
    }
    __syncthreads();
  }
  return S;
}

// Rescan the chosen tile: the same weights and per-lane fp32 sums as its tile
// sum, fp64 prefix.  Writes y, C_{y-1} and C_y (unnormalised) and pi(y)'s
// weight recomputed with the precise residual.
template <int DT, bool VEC, int MODE>
__device__ int rescan_tile(const VerifyArgs& a, int b, int k, const SampleCoef& cf, double target,
                           RefineLds& sh) {
  const int tid = threadIdx.x;
  const int tsel = sh.tile;
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  const int64_t j0 = (int64_t)tsel * kTile + (int64_t)tid * kUnit;
  Raw8<DT, VEC> rd, rt;
  load_raw<DT, VEC>(trow, j0, a.V, rt);
  if constexpr (MODE != kModeTarget) load_raw<DT, VEC>(drow, j0, a.V, rd);
  float ld[8], lt[8], w[8], r[8];
  unpack<DT, VEC>(rt, lt);
  if constexpr (MODE != kModeTarget) unpack<DT, VEC>(rd, ld);
  sample_weights<DT, MODE, false>(ld, lt, cf, w, r);
  float ws = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ws += w[e];
  double tile_tot;
  const double off = block_exclusive_scan((double)ws, sh.lds_d, tile_tot);
  const double tgt = target - sh.off;
  int cand = INT_MAX;
  if (off <= tgt && tgt < off + (double)ws) {
    double run = off;
    bool found = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double nx = run + (double)w[e];
      if (!found && w[e] > 0.f && tgt < nx) {
        cand = (int)(j0 + e);
        found = true;
      }
      run = nx;
    }
  }
  int y = block_min_int(cand, sh.lds_i);
  if (y == INT_MAX) {   // rounding left the target past every running sum: last token with weight
    int last = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (w[e] > 0.f) last = (int)(j0 + e);
    y = -block_min_int(-last, sh.lds_i);
    if (y < 0) y = (int)min<int64_t>(a.V - 1, (int64_t)tsel * kTile + kTile - 1);
  }
  if (y >= j0 && y < j0 + 8) {   // the owner of y reports C_{y-1}, C_y and pi(y)
    const int idx = (int)(y - j0);
    double run = sh.off + off, wy = 0.0;
    float ldy = 0.f, lty = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e < idx) run += (double)w[e];
      if (e == idx) {
        wy = (double)w[e];
        ldy = ld[e];
        lty = lt[e];
      }
    }
    sh.lo = run;
    sh.hi = run + wy;
    float rr;
    sh.w = (double)weight_rt<DT, true>(MODE, ldy, lty, cf, rr);
  }
  __syncthreads();
  return y;
}

// Locate, rescan and write the outputs (run by the last pass-B item).
template <int DT, bool VEC>
__device__ void refine_seq(const VerifyArgs& a, int b, RefineLds& sh) {
  const int tid = threadIdx.x;
  const SeqRec rec = load_rec(a.seq + b);
  if (!rec.valid) return;   // outputs were written by the decision
  const int g = a.gamma, k = rec.k;
  const int64_t orow = (int64_t)b * (g + 1);
  double* tiles = a.tiles + (int64_t)b * a.ntile;
  const SampleCoef cf = coef_of(a, rec);
  int mode = rec.mode;
  if (tid == 0) sh.tile = -1;

  double rtot = 0.0;
  for (int i = tid; i < a.nt; i += kThreads) rtot += ld_dev(a.itemsum + (int64_t)b * a.nt + i);
  rtot = block_sum(rtot, sh.lds_d);
  if (mode == kModeTarget) rtot = 0.0;

  const double u = (double)a.u_smp[orow + k];
  double target = 0.0;
  double S = locate_tile(tiles, a.ntile, u, sh, target);
  while (!(S > 0.0) && mode != kModeTarget) {
    // A zero Saguaro normaliser falls back to the residual, a zero residual
    // mass to q_k: recompute every tile sum here (degenerate inputs only).
    mode = mode == kModeResidual ? kModeTarget : kModeResidual;
    if (mode == kModeTarget) rtot = 0.0;
    const void *drow, *trow;
    draw_rows<DT>(a, b, k, drow, trow);
    for (int t = 0; t < a.ntile; ++t) {
      float ws = 0.f;
#pragma unroll 1
      for (int e = 0; e < kUnit; ++e) {
        const int64_t j = (int64_t)t * kTile + (int64_t)tid * kUnit + e;
        float rr;
        if (j < a.V)
          ws += weight_rt<DT, false>(mode, load_one<DT>(drow, j), load_one<DT>(trow, j), cf, rr);
      }
      const double tw = block_sum((double)ws, sh.lds_d);
      if (tid == 0) st_dev(tiles + t, tw);
    }
    if (tid == 0) {
      wait_mem();
      sh.tile = -1;
    }
    __syncthreads();
    S = locate_tile(tiles, a.ntile, u, sh, target);
  }

  int y = 0;
  with_mode(mode, [&](auto m) { y = rescan_tile<DT, VEC, decltype(m)::value>(a, b, k, cf, target, sh); });

  if (tid <= g) {
    int tok = -1;
    if (tid < k) tok = a.tokens[(int64_t)b * g + tid];
    else if (tid == k) tok = y;
    a.out_tokens[orow + tid] = tok;
  }
  if (tid == 0) {
    a.out_acc[b] = k;
    if (a.out_first_reject) a.out_first_reject[b] = k < g ? k : -1;
    if (a.out_mask) a.out_mask[b] = rec.mask;
    if (a.out_len) a.out_len[b] = (a.in_len ? a.in_len[b] : 0) + k + 1;
    if (a.diag.resid_mass) a.diag.resid_mass[b] = k < g ? rtot / rec.Zt : 0.0;
    if (a.diag.token_prob) a.diag.token_prob[b] = sh.w / S;
    if (a.diag.cdf_lo) a.diag.cdf_lo[b] = sh.lo / S;
    if (a.diag.cdf_hi) a.diag.cdf_hi[b] = sh.hi / S;
  }
}

// ---------------------------------------------------------------------------
// Kernels.

template <int DT, bool VEC, int U, bool DECIDE>
__global__ __launch_bounds__(kThreads) void stream_kernel(VerifyArgs a) {
  __shared__ float lds_f[2 * kWaves];
  __shared__ double lds_d[kWaves];
  const int R = 2 * a.gamma + 1;
  const int64_t id = blockIdx.x;
  const int per_seq = R * a.nc;
  const int b = (int)(id / per_seq);
  const int rem = (int)(id - (int64_t)b * per_seq);
  const int r = rem / a.nc, c = rem - r * a.nc;
  stream_item<DT, VEC, U>(a, b, r, c, lds_f, lds_d);
  if constexpr (DECIDE) {
    __shared__ int flag;
    __shared__ DecideLds dsh;
    if (arrive(&a.ctr[b].stream_done, (unsigned)per_seq, &flag)) decide_seq<DT>(a, b, dsh);
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void decide_kernel(VerifyArgs a) {
  __shared__ DecideLds dsh;
  decide_seq<DT>(a, blockIdx.x, dsh);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_a_kernel(VerifyArgs a) {
  __shared__ double lds_d[kWaves * (kTilesPerItem + 1)];
  __shared__ int flag;
  const int b = blockIdx.x / a.nt, s = blockIdx.x - b * a.nt;
  sample_item_a<DT, VEC>(a, b, s, lds_d);
  if (arrive(&a.ctr[b].a_done, (unsigned)a.nt, &flag)) finish_a(a, b, lds_d);
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void sample_b_kernel(VerifyArgs a) {
  __shared__ RefineLds sh;
  __shared__ int flag;
  const int b = blockIdx.x / a.nt, s = blockIdx.x - b * a.nt;
  sample_item_b<DT, VEC>(a, b, s, sh.lds_d);
  if (arrive(&a.ctr[b].b_done, (unsigned)a.nt, &flag)) refine_seq<DT, VEC>(a, b, sh);
}

// ---------------------------------------------------------------------------
// Fused persistent kernel.
//
// Items are numbered in steps: step t holds the stream items of sequence t,
// then the residual-mass items (Saguaro eps > 0) of sequence t - LA, then the
// sampling items of sequence t - LB.  Work-groups take item numbers in
// increasing order from a global counter (one item ahead, so the atomic's
// latency overlaps the current item), so items run nearly in order and a
// sequence's sampling items start about LB steps after its rows were
// streamed, re-reading them from the 256 MB last-level cache.  A sampling
// item waits (bounded spin) for its sequence's decision, which the last of
// the sequence's stream items makes.  An item waits only on items with
// smaller numbers, all of them already taken by resident work-groups (the
// launch is cooperative), so the smallest unfinished item can always run.

struct Sched {
  int B, NS, NA, NB, LA, LB;
  int64_t total;
};

__host__ __device__ inline int64_t sched_offset(const Sched& s, int t) {
  const int ns = t < s.B ? t : s.B;
  int na = t - s.LA, nb = t - s.LB;
  na = na < 0 ? 0 : (na > s.B ? s.B : na);
  nb = nb < 0 ? 0 : (nb > s.B ? s.B : nb);
  return (int64_t)ns * s.NS + (int64_t)na * s.NA + (int64_t)nb * s.NB;
}

enum : int { kItemStream = 0, kItemA = 1, kItemB = 2 };

__device__ __forceinline__ void sched_decode(const Sched& s, int64_t j, int& kind, int& b, int& sub) {
  int lo = 0, hi = s.B + s.LB;   // offset(lo) <= j < offset(hi) = total
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (sched_offset(s, mid) <= j) lo = mid;
    else hi = mid;
  }
  int64_t w = j - sched_offset(s, lo);
  if (lo < s.B) {
    if (w < s.NS) {
      kind = kItemStream;
      b = lo;
      sub = (int)w;
      return;
    }
    w -= s.NS;
  }
  const int ba = lo - s.LA;
  if (s.NA > 0 && ba >= 0 && ba < s.B) {
    if (w < s.NA) {
      kind = kItemA;
      b = ba;
      sub = (int)w;
      return;
    }
    w -= s.NA;
  }
  kind = kItemB;
  b = lo - s.LB;
  sub = (int)w;
}

// Bounded spin until *flag is nonzero (thread 0 polls; the work-group follows).
// A timeout records an error instead of hanging.
__device__ __forceinline__ void wait_flag(const VerifyArgs& a, unsigned* flag, int* lds_flag) {
  if (threadIdx.x == 0) {
    unsigned polls = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      __builtin_amdgcn_s_sleep(2);
      if (++polls > (1u << 23)) {   // about half a second
        __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    *lds_flag = 0;
  }
  __syncthreads();
}

__device__ __forceinline__ void set_flag(unsigned* flag) {
  if (threadIdx.x == 0) {
    wait_mem();
    __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(SV_FUSED_WAVES, SV_FUSED_WAVES)))
void fused_kernel(VerifyArgs a, Sched sc) {
  __shared__ union {
    DecideLds d;
    RefineLds r;
  } sh;
  __shared__ float lds_f[2 * kWaves];
  __shared__ double lds_d[kWaves * (kTilesPerItem + 1)];
  __shared__ int flag;
  __shared__ unsigned item;
  const bool eps_mode = a.saguaro && a.eps > 0.f;
  const unsigned grabs = (unsigned)sc.total + gridDim.x;   // every work-group over-takes once
  unsigned ahead = 0;
  if (threadIdx.x == 0)
    ahead = __hip_atomic_fetch_add(a.next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (;;) {
    if (threadIdx.x == 0) {
      item = ahead;
      if (ahead == grabs - 1)   // the last take of the call: leave the counter zeroed
        __hip_atomic_store(a.next, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else if (ahead < sc.total)
        ahead = __hip_atomic_fetch_add(a.next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int64_t j = item;
    if (j >= sc.total) break;
    int kind, b, sub;
    sched_decode(sc, j, kind, b, sub);
    SeqCtr& ctr = a.ctr[b];
    if (kind == kItemStream) {
      const int r = sub / a.nc, c = sub - r * a.nc;
      stream_item<DT, VEC, U>(a, b, r, c, lds_f, lds_d);
      if (arrive(&ctr.stream_done, (unsigned)sc.NS, &flag)) {
        decide_seq<DT>(a, b, sh.d);
        __syncthreads();
        set_flag(&ctr.decided);
      }
    } else if (kind == kItemA) {
      wait_flag(a, &ctr.decided, &flag);
      sample_item_a<DT, VEC>(a, b, sub, lds_d);
      if (arrive(&ctr.a_done, (unsigned)a.nt, &flag)) {
        finish_a(a, b, lds_d);
        __syncthreads();
        set_flag(&ctr.a_ready);
      }
    } else {
      wait_flag(a, eps_mode ? &ctr.a_ready : &ctr.decided, &flag);
      sample_item_b<DT, VEC>(a, b, sub, lds_d);
      if (arrive(&ctr.b_done, (unsigned)a.nt, &flag)) {
        refine_seq<DT, VEC>(a, b, sh.r);
        if (threadIdx.x == 0) {   // every reader of the flags has passed them
          __hip_atomic_store(&ctr.decided, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&ctr.a_ready, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host side.

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  int nc, chunk, ntile, nt;
  size_t err_off, part_off, seq_off, ctr_off, tiles_off, item_off, total;
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
  off += align256((size_t)B * R * L.nc * sizeof(Partial));
  L.seq_off = off;
  off += align256((size_t)B * sizeof(SeqRec));
  L.ctr_off = off;
  off += align256((size_t)B * sizeof(SeqCtr));
  L.tiles_off = off;
  off += align256((size_t)B * L.ntile * sizeof(double));
  L.item_off = off;
  off += align256((size_t)B * L.nt * sizeof(double));
  L.total = B == 0 ? 0 : off;
  return L;
}

template <int DT, bool VEC>
static hipError_t launch_all(const VerifyArgs& a, hipStream_t st) {
  const int R = 2 * a.gamma + 1;
  if (SV_FUSED) {
    auto kern = fused_kernel<DT, VEC, SV_STREAM_UNROLL>;
    int dev = 0, ncu = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                       kThreads, 0);
    if (e != hipSuccess) return e;
    Sched sc;
    sc.B = a.B;
    sc.NS = R * a.nc;
    sc.NA = (a.saguaro && a.eps > 0.f) ? a.nt : 0;
    sc.NB = a.nt;
    const int64_t all = (int64_t)a.B * (sc.NS + sc.NA + sc.NB);
    const int64_t G = std::max<int64_t>(1, std::min<int64_t>((int64_t)per_cu * ncu, all));
    const int64_t per_step = sc.NS + sc.NA + sc.NB;
    const int L = (int)std::max<int64_t>(1, (G * SV_LAG_MILLIROUNDS / 1000 + per_step - 1) / per_step);
    sc.LA = L;
    sc.LB = sc.NA > 0 ? 2 * L : L;
    sc.total = all;
    VerifyArgs args = a;
    void* params[] = {&args, &sc};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3((unsigned)G),
                                      dim3(kThreads), params, 0, st);
  }
  const unsigned nstream = (unsigned)((int64_t)a.B * R * a.nc);
  const unsigned nsample = (unsigned)((int64_t)a.B * a.nt);
  hipLaunchKernelGGL((stream_kernel<DT, VEC, SV_STREAM_UNROLL, false>), dim3(nstream), dim3(kThreads),
                     0, st, a);
  hipLaunchKernelGGL((decide_kernel<DT>), dim3((unsigned)a.B), dim3(kThreads), 0, st, a);
  if (a.saguaro && a.eps > 0.f)
    hipLaunchKernelGGL((sample_a_kernel<DT, VEC>), dim3(nsample), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((sample_b_kernel<DT, VEC>), dim3(nsample), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

static int verify_impl(const void* draft, const void* target, int dtype, const int32_t* tokens,
                       const float* u_acc, const float* u_smp, int B, int gamma, int V, float T,
                       const int32_t* in_len, int32_t* out_tokens, int32_t* out_acc,
                       int32_t* out_fr, uint64_t* out_mask, int32_t* out_len,
                       const spec_diag* diag, void* ws, size_t ws_bytes, void* stream,
                       int saguaro, float eps) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (!sizes_ok(B, gamma, V)) return SPEC_EINVAL;
  if (!(T > 0.f) || !std::isfinite(T)) return SPEC_EINVAL;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!draft || !target || !tokens || !u_acc || !u_smp || !out_tokens || !out_acc)
    return SPEC_EINVAL;
  const Layout L = layout(B, gamma, V);
  // Grid limit: at most 2^32 - 1 work-items per launch dimension.
  if ((int64_t)B * (2 * gamma + 1) * L.nc * kThreads > (int64_t)UINT_MAX) return SPEC_EINVAL;
  if ((int64_t)B * L.nt * kThreads > (int64_t)UINT_MAX) return SPEC_EINVAL;
  // Fused item numbers (plus one extra take per work-group) fit in 32 bits.
  if ((int64_t)B * ((2 * gamma + 1) * L.nc + 2 * L.nt) > (int64_t)INT_MAX / 2) return SPEC_EINVAL;
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
  a.next = reinterpret_cast<unsigned*>(w + L.err_off + 8);
  a.part = reinterpret_cast<Partial*>(w + L.part_off);
  a.seq = reinterpret_cast<SeqRec*>(w + L.seq_off);
  a.ctr = reinterpret_cast<SeqCtr*>(w + L.ctr_off);
  a.tiles = reinterpret_cast<double*>(w + L.tiles_off);
  a.itemsum = reinterpret_cast<double*>(w + L.item_off);
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

  const bool vec = (V % 8 == 0) && ((uintptr_t)draft % 16 == 0) && ((uintptr_t)target % 16 == 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e;
  if (dtype == SPEC_BF16) e = vec ? launch_all<kBF16, true>(a, st) : launch_all<kBF16, false>(a, st);
  else e = vec ? launch_all<kF32, true>(a, st) : launch_all<kF32, false>(a, st);
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
