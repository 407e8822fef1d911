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

constexpr int kTilesPerItem = 4;

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

// Arrival counters of one sequence, one 128-byte line each.
struct SeqCtr {
  unsigned stream_done;
  unsigned a_done;
  unsigned b_done;
  unsigned pad[29];
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
  for (int64_t j = begin + (int64_t)threadIdx.x * kUnit; j < end; j += kStep * U) {
    float v[U * 8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ju = j + u * kStep;
      float(&vu)[8] = *reinterpret_cast<float(*)[8]>(v + u * 8);
      if (ju < end) {
        load8<DT, VEC>(row, ju, end, vu);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vu[e] = -INFINITY;
      }
    }
    float bm = v[0];
#pragma unroll
    for (int e = 1; e < U * 8; ++e) bm = fmaxf(bm, v[e]);
    mraw = fmaxf(mraw, bm);
    const float bl = bm * ch;
    if (bl > mref) {   // new offset: rescale the running sum by an exact power of two
      const float nref = ceilf(fminf(bl, 1.0e30f));
      if (s != 0.0) s = ldexp(s, (int)fmaxf(mref - nref, -2000.f));
      mref = nref;
    }
#pragma unroll
    for (int e = 0; e < U * 8; ++e) v[e] = exp2_fast(fmaf(v[e], cl, fmaf(v[e], ch, -mref)));
#pragma unroll
    for (int w = U * 4; w >= 1; w >>= 1)   // pairwise sum of the batch in fp32
#pragma unroll
      for (int e = 0; e < w; ++e) v[e] += v[e + w];
    s += (double)v[0];
  }
  const float mb = block_max(mref, lds_f);
  const float mr = block_max(mraw, lds_f);
  const double sd = (s != 0.0) ? ldexp(s, (int)fmaxf(mref - mb, -2000.f)) : 0.0;
  const double sb = block_sum(sd, lds_d);
  if (threadIdx.x == 0)
    store_partial(a.part + ((int64_t)b * (2 * a.gamma + 1) + r) * a.nc + c, mb, mr, sb);
}

// ---------------------------------------------------------------------------
// Decision of one sequence (run by its last stream item).

struct DecideLds {
  float M[128];
  double Z[128];
  int bad[128];
  uint64_t mask;
  int k, valid;
};

template <int DT>
__device__ void decide_seq(const VerifyArgs& a, int b, DecideLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = a.gamma, R = 2 * g + 1;
  const double cTd = a.cTd;
  const Partial* P0 = a.part + (int64_t)b * R * a.nc;

  // 1. Merge each row's chunk pieces (one wave per row, lanes over chunks; fp64).
  for (int r = wave; r < R; r += kWaves) {
    const Partial* P = P0 + (int64_t)r * a.nc;
    float M = kNegSentinel, mr = -INFINITY;
    // lanes hold their chunks' pieces (nc <= 64 in one pass; more loop)
    for (int c0 = 0; c0 < a.nc; c0 += 64) {
      const int c = c0 + lane;
      const Partial p = c < a.nc ? load_partial(P + c) : Partial{kNegSentinel, -INFINITY, 0.0};
      M = fmaxf(M, p.mc);
      mr = fmaxf(mr, p.mraw);
    }
    M = wave_max(M);
    mr = wave_max(mr);
    double z = 0.0;
    for (int c0 = 0; c0 < a.nc; c0 += 64) {
      const int c = c0 + lane;
      const Partial p = c < a.nc ? load_partial(P + c) : Partial{kNegSentinel, -INFINITY, 0.0};
      if (p.s != 0.0) z += ldexp(p.s, (int)fmaxf(p.mc - M, -2000.f));
    }
    z = wave_sum(z);
    if (lane == 0) {
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

  // 2. Accept test at every draft position (wave 0, lane i = position i).
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
    a.seq[b] = rec;
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

// 1 - 2^d for d in (-1, 0]: -expm1(d ln 2) by its Taylor series (degree 9,
// truncation below 1e-8 relative); 1 - 2^d directly for d <= -1.
__device__ __forceinline__ float one_minus_exp2(float d, float ex) {
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

// Sampling weights of eight logits, each proportional (one factor per
// sequence) to the probability of the distribution drawn from:
//   target row:  q_j                      (eq_j = 2^(lt_j c_T - Mt))
//   residual:    (q_j - p_j)+             (eq_j (1 - 2^delta_j) where delta_j < 0)
//   Saguaro:     sqrt(p_j (q_j - p_j)+)   (eq_j sqrt(2^delta_j (1 - 2^delta_j)))
//   Saguaro eps: sqrt(p_j max(r_j, eps))  (sqrt(eq_j 2^delta_j max(res_j, eps sum res)))
// with delta_j = log2(p_j / q_j) = (ld_j - lt_j) c_T + K.  The residual is
// formed from delta_j (exact logit difference for bf16, a two-sum for
// float32), so its relative error stays at a few ulp where q_j and p_j nearly
// cancel.  r = the residual weight.
template <int DT>
__device__ __forceinline__ void sample_weights(int mode, const float (&ld)[8], const float (&lt)[8],
                                               const SampleCoef& c, float (&w)[8], float (&r)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float eq = exp2_fast(fmaf(lt[e], c.c_lo, fmaf(lt[e], c.c_hi, -c.Mt)));
    if (mode == kModeTarget) {
      w[e] = eq;
      r[e] = 0.f;
      continue;
    }
    const float dl = ld[e] - lt[e];
    float d;
    if constexpr (DT == kBF16) {
      d = fmaf(dl, c.c_hi, c.K_hi) + fmaf(dl, c.c_lo, c.K_lo);   // dl is exact
    } else {
      const float bb = dl - ld[e];
      const float err = (ld[e] - (dl - bb)) - (lt[e] + bb);       // ld - lt = dl + err
      d = fmaf(dl, c.c_hi, c.K_hi) + fmaf(err, c.c_hi, fmaf(dl, c.c_lo, c.K_lo));
    }
    const float ex = exp2_fast(d);          // p_j / q_j
    const float em1 = one_minus_exp2(d, ex);
    const bool pos = (eq > 0.f) && (d < 0.f);
    const float res = pos ? eq * em1 : 0.f;
    r[e] = res;
    if (mode == kModeResidual) w[e] = res;
    else if (mode == kModeSaguaro) w[e] = pos ? eq * sqrtf(ex * em1) : 0.f;
    else w[e] = (eq > 0.f) ? sqrtf(eq * ex * fmaxf(res, c.epsS)) : 0.f;
  }
}

template <int DT, bool VEC>
__device__ __forceinline__ void load_pair(int mode, const void* drow, const void* trow, int64_t j0,
                                          int64_t V, float (&ld)[8], float (&lt)[8]) {
  if (j0 < V) {
    load8<DT, VEC>(trow, j0, V, lt);
    if (mode != kModeTarget) load8<DT, VEC>(drow, j0, V, ld);
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

// Tile sums of the weights of `mode` over tiles [t0, t0 + kTilesPerItem) (clipped
// to ntile): tw[i] (fp64, identical in every thread) and the residual total.
template <int DT, bool VEC>
__device__ __forceinline__ void tile_sums(const VerifyArgs& a, int b, int mode, const SampleCoef& cf,
                                          int k, int t0, double (&tw)[kTilesPerItem + 1],
                                          double* lds_d) {
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  const int64_t lane_off = (int64_t)threadIdx.x * kUnit;
  float ld[kTilesPerItem][8], lt[kTilesPerItem][8];
#pragma unroll
  for (int i = 0; i < kTilesPerItem; ++i) {
    const int t = t0 + i;
    const int64_t j0 = t < a.ntile ? (int64_t)t * kTile + lane_off : (int64_t)a.V;
    load_pair<DT, VEC>(mode, drow, trow, j0, a.V, ld[i], lt[i]);
  }
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < kTilesPerItem; ++i) {
    float w[8], r[8];
    sample_weights<DT>(mode, ld[i], lt[i], cf, w, r);
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
  const SeqRec rec = a.seq[b];
  double tw[kTilesPerItem + 1] = {0, 0, 0, 0, 0};
  if (rec.valid && rec.mode == kModeSaguaroEps)
    tile_sums<DT, VEC>(a, b, kModeResidual, coef_of(a, rec), rec.k, s * kTilesPerItem, tw, lds_d);
  if (threadIdx.x == 0) st_dev(a.itemsum + (int64_t)b * a.nt + s, tw[kTilesPerItem]);
}

// eps * residual mass, by the last pass-A item of a sequence.
__device__ void finish_a(const VerifyArgs& a, int b, double* lds_d) {
  double v = 0.0;
  for (int i = threadIdx.x; i < a.nt; i += kThreads) v += ld_dev(a.itemsum + (int64_t)b * a.nt + i);
  v = block_sum(v, lds_d);
  if (threadIdx.x == 0) a.seq[b].epsS = (float)(v * (double)a.eps);
}

// Tile sums of the sampling weights (pass B).
template <int DT, bool VEC>
__device__ void sample_item_b(const VerifyArgs& a, int b, int s, double* lds_d) {
  const SeqRec rec = a.seq[b];
  if (!rec.valid) return;
  double tw[kTilesPerItem + 1];
  const int t0 = s * kTilesPerItem;
  tile_sums<DT, VEC>(a, b, rec.mode, coef_of(a, rec), rec.k, t0, tw, lds_d);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < kTilesPerItem; ++i)
      if (t0 + i < a.ntile) st_dev(a.tiles + (int64_t)b * a.ntile + t0 + i, tw[i]);
    st_dev(a.itemsum + (int64_t)b * a.nt + s, tw[kTilesPerItem]);
  }
}

struct RefineLds {
  double lds_d[kWaves * (kTilesPerItem + 1)];
  int lds_i[kWaves];
  int tile;
  double off, lo, hi, w;
};

// Locate, rescan and write the outputs (run by the last pass-B item).
template <int DT, bool VEC>
__device__ void refine_seq(const VerifyArgs& a, int b, RefineLds& sh) {
  const int tid = threadIdx.x;
  const SeqRec rec = a.seq[b];
  if (!rec.valid) return;   // outputs were written by the decision
  const int g = a.gamma, k = rec.k;
  const int64_t orow = (int64_t)b * (g + 1);
  double* tiles = a.tiles + (int64_t)b * a.ntile;
  SampleCoef cf = coef_of(a, rec);
  int mode = rec.mode;

  double rtot = 0.0;
  for (int i = tid; i < a.nt; i += kThreads) rtot += ld_dev(a.itemsum + (int64_t)b * a.nt + i);
  rtot = block_sum(rtot, sh.lds_d);
  if (mode == kModeTarget) rtot = 0.0;

  double S = 0.0;
  for (;;) {
    double v = 0.0;
    for (int i = tid; i < a.ntile; i += kThreads) v += ld_dev(tiles + i);
    S = block_sum(v, sh.lds_d);
    if (S > 0.0 || mode == kModeTarget) break;
    // A zero Saguaro normaliser falls back to the residual, a zero residual
    // mass to q_k: recompute every tile sum here (degenerate inputs only).
    mode = mode == kModeResidual ? kModeTarget : kModeResidual;
    if (mode == kModeTarget) rtot = 0.0;
    for (int t0 = 0; t0 < a.ntile; t0 += kTilesPerItem) {
      double tw[kTilesPerItem + 1];
      tile_sums<DT, VEC>(a, b, mode, cf, k, t0, tw, sh.lds_d);
      if (tid == 0)
        for (int i = 0; i < kTilesPerItem; ++i)
          if (t0 + i < a.ntile) st_dev(tiles + t0 + i, tw[i]);
    }
    if (tid == 0) wait_mem();
    __syncthreads();
  }

  // Tile holding u * S: fp64 exclusive scan over the tile sums in token order.
  const double target = (double)a.u_smp[orow + k] * S;
  if (tid == 0) sh.tile = -1;
  __syncthreads();
  double carry = 0.0;
  for (int base = 0; base < a.ntile; base += kThreads) {
    const int t = base + tid;
    const double v = t < a.ntile ? ld_dev(tiles + t) : 0.0;
    double tot;
    const double off = carry + block_exclusive_scan(v, sh.lds_d, tot);
    // Intervals of nonzero tiles are disjoint up to rounding: take the first.
    const int hit = (t < a.ntile && off <= target && target < off + v) ? t : INT_MAX;
    const int first = block_min_int(hit, sh.lds_i);
    if (first != INT_MAX) {
      if (t == first) {
        sh.tile = t;
        sh.off = off;
      }
      __syncthreads();
      break;
    }
    carry += tot;
  }
  if (sh.tile < 0) {   // u * S at or past the last running sum (rounding): last nonzero tile
    int last = -1;
    for (int t = tid; t < a.ntile; t += kThreads)
      if (ld_dev(tiles + t) > 0.0) last = t;
    last = -block_min_int(-last, sh.lds_i);
    if (tid == 0) {
      sh.tile = last;
      double off = 0.0;
      for (int t = 0; t < last; ++t) off += ld_dev(tiles + t);
      sh.off = off;
    }
    __syncthreads();
  }

  // Rescan the tile: the same per-lane fp32 sums, fp64 prefix.
  const int tsel = max(sh.tile, 0);
  const void *drow, *trow;
  draw_rows<DT>(a, b, k, drow, trow);
  const int64_t j0 = (int64_t)tsel * kTile + (int64_t)tid * kUnit;
  float ld[8], lt[8], w[8], r[8];
  load_pair<DT, VEC>(mode, drow, trow, j0, a.V, ld, lt);
  sample_weights<DT>(mode, ld, lt, cf, w, r);
  float ws = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ws += w[e];
  double tile_tot;
  const double off = block_exclusive_scan((double)ws, sh.lds_d, tile_tot);
  const double tgt = target - sh.off;
  int cand = INT_MAX;
  if (off <= tgt && tgt < off + (double)ws) {
    double run = off;
    for (int e = 0; e < 8; ++e) {
      const double nx = run + (double)w[e];
      if (w[e] > 0.f && tgt < nx) {
        cand = (int)(j0 + e);
        break;
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
    double run = sh.off + off;
    for (int e = 0; e < (int)(y - j0); ++e) run += (double)w[e];
    sh.lo = run;
    sh.w = (double)w[y - j0];
    sh.hi = run + (double)w[y - j0];
  }
  __syncthreads();

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

template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kThreads) void stream_kernel(VerifyArgs a) {
  __shared__ float lds_f[kWaves];
  __shared__ double lds_d[kWaves];
  __shared__ int flag;
  __shared__ DecideLds dsh;
  const int R = 2 * a.gamma + 1;
  const int64_t id = blockIdx.x;
  const int per_seq = R * a.nc;
  const int b = (int)(id / per_seq);
  const int rem = (int)(id - (int64_t)b * per_seq);
  const int r = rem / a.nc, c = rem - r * a.nc;
  stream_item<DT, VEC, U>(a, b, r, c, lds_f, lds_d);
  if (arrive(&a.ctr[b].stream_done, (unsigned)per_seq, &flag)) decide_seq<DT>(a, b, dsh);
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
// Host side.

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  int nc, chunk, ntile, nt;
  size_t part_off, seq_off, ctr_off, tiles_off, item_off, total;
};

static bool sizes_ok(int B, int gamma, int V) {
  return B >= 0 && gamma >= 1 && gamma <= 63 && V >= 1;
}

static Layout layout(int B, int gamma, int V) {
  Layout L;
  const int nc0 = (V + kChunk - 1) / kChunk;
  L.chunk = (int)((((int64_t)V + nc0 - 1) / nc0 + 7) / 8 * 8);   // balanced, a multiple of 8
  L.nc = (int)(((int64_t)V + L.chunk - 1) / L.chunk);
  L.ntile = (V + kTile - 1) / kTile;
  L.nt = (L.ntile + kTilesPerItem - 1) / kTilesPerItem;
  const size_t R = 2 * (size_t)gamma + 1;
  size_t off = 0;
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
static void launch_all(const VerifyArgs& a, hipStream_t st) {
  const int R = 2 * a.gamma + 1;
  const unsigned nstream = (unsigned)((int64_t)a.B * R * a.nc);
  const unsigned nsample = (unsigned)((int64_t)a.B * a.nt);
  hipLaunchKernelGGL((stream_kernel<DT, VEC, 4>), dim3(nstream), dim3(kThreads), 0, st, a);
  if (a.saguaro && a.eps > 0.f)
    hipLaunchKernelGGL((sample_a_kernel<DT, VEC>), dim3(nsample), dim3(kThreads), 0, st, a);
  hipLaunchKernelGGL((sample_b_kernel<DT, VEC>), dim3(nsample), dim3(kThreads), 0, st, a);
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
  if (dtype == SPEC_BF16) {
    if (vec) launch_all<kBF16, true>(a, st);
    else launch_all<kBF16, false>(a, st);
  } else {
    if (vec) launch_all<kF32, true>(a, st);
    else launch_all<kF32, false>(a, st);
  }
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
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
