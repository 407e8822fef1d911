// Sampling: weights, residual-mass, sampling, draw and final items.
#pragma once
#include "verify_decide.h"
#undef SV_FILE
#define SV_FILE 4

namespace sv {

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
    const int64_t t0 = (int64_t)b * (2 * a.gamma + 1);
    c.Lt = uni(SV_AT(a, topp, t0 + (a.gamma + rec.k))->L);
    if (rec.k < a.gamma) c.Ld = uni(SV_AT(a, topp, t0 + rec.k)->L);
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
// A slot whose wait gave up reads as NaN, so the clamp is NaN then.
__device__ float eps_clamp(const VerifyArgs& a, int b, double* lds_d) {
  double v = 0.0;
  for (int i = threadIdx.x; i < a.nt; i += kThreads) v += slot_value(poll(a, SV_AT(a, mass, (int64_t)b * a.nt + i)));
  v = block_sum(v, lds_d);
  return uni((float)(v * (double)a.eps));
}

// ---------------------------------------------------------------------------
// Residual-mass and sampling items.

// N tiles per item, as the call's sampling items take.
template <int DT, bool VEC, bool CUT = false, int N = kTilesPerItem>
__device__ __forceinline__ void mass_item(const VerifyArgs& a, int b, int s, double* lds_d) {
  const SeqRec rec = wait_rec<true>(a, b);
  if (!rec.valid || rec.mode != kModeSaguaroEps) return;
  double tw[N + 1];
  float mt[N];
  tile_sums<DT, VEC, kModeResidual, CUT, N>(a, b, coef_of<CUT>(a, b, rec, 0.f), rec.k, s * N, tw, mt, lds_d);
  if (threadIdx.x == 0) slot_put(SV_AT(a, mass, (int64_t)b * a.nt + s), tw[N]);
}

// N tiles per item (kTilesPerItem, or fewer for short calls: see
// sample_tiles); a.nt items per sequence.
template <int DT, bool VEC, bool CUT = false, bool EPS = true, int N = kTilesPerItem>
__device__ __forceinline__ void sample_item(const VerifyArgs& a, int b, int s, double* lds_d) {
  static_assert(N >= 1 && N <= kTilesPerItem, "the LDS of a sampling item holds kTilesPerItem tiles");
  const SeqRec rec = wait_rec<true>(a, b);
  if (!rec.valid) return;
  const int t0 = (int)SV_IDX(a, s * N, a.ntile);
  const float epsS = rec.mode == kModeSaguaroEps ? eps_clamp(a, b, lds_d) : 0.f;
  const SampleCoef cf = coef_of<CUT>(a, b, rec, epsS);
  with_mode<EPS>(rec.mode, [&](auto m) {
    constexpr int MODE = decltype(m)::value;
    double tw[N + 1];
    float mt[N];
    tile_sums<DT, VEC, MODE, CUT, N>(a, b, cf, rec.k, t0, tw, mt, lds_d);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int i = 0; i < N; ++i)
        if (t0 + i < a.ntile)
          slot_put(SV_AT(a, tiles, (int64_t)b * a.ntile + t0 + i), tile_slot_value(MODE, tw[i], mt[i]));
      if (MODE == kModeSaguaro) slot_put(SV_AT(a, rsum, (int64_t)b * a.nt + s), tw[N]);
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
  double w8d[kUnit];                 // fp64 residual draw: the owner lane's weights
  double n_rm, n_tp, n_lo, n_hi;     // fp64 residual draw: S, pi(y), C_{y-1}, C_y (normalised)
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

// locate_tile for at most kThreads tiles whose values the threads already
// hold: thread t passes tile t's value v (0 past ntile).  The same scan, and
// the same tile and offset, without reading the slots again.
__device__ double locate_tile_held(double v, int ntile, double u, DrawLds& sh, double& target) {
  const int tid = threadIdx.x;
  double tot;
  const double off = block_exclusive_scan(v, sh.lds_d, tot);
  const double S = tot;
  target = u * S;
  const int hit = (tid < ntile && off <= target && target < off + v) ? tid : INT_MAX;
  const int first = block_min_int(hit, sh.lds_i);
  if (first != INT_MAX) {
    if (tid == first) {
      sh.tile = tid;
      sh.off = off;
    }
  } else {   // u * S at or past the last running sum (rounding): the last tile with mass
    const int last = -block_min_int((tid < ntile && v > 0.0) ? -tid : 1, sh.lds_i);
    if (tid == max(last, 0)) {
      sh.tile = max(last, 0);
      sh.off = last > 0 ? off : 0.0;
    }
  }
  __syncthreads();
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
__device__ __forceinline__ void rescan_tile(const VerifyArgs& a, int b, int k, const SampleCoef& cf, double target,
                            DrawLds& sh) {
  const int tid = threadIdx.x;
  const int tsel = (int)SV_IDX(a, sh.tile, a.ntile);
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
  y = (int)SV_IDX(a, y, a.V);
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
__device__ __forceinline__ void recompute_tiles(const VerifyArgs& a, int b, int k, int mode, const SampleCoef& cf,
                                DrawLds& sh) {
  uint64_t* tiles = SV_AT(a, tiles, (int64_t)b * a.ntile);
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

// ---------------------------------------------------------------------------
// Residual draws refined in fp64.
//
// The fp32 weights (q_j - p_j)+ of the sampling items carry an absolute error
// of a few ulp of q_j and p_j, and the row normalisers from the stream a
// relative error of the same order, so the running sums of the residual are
// known to some 1e-8 of q_k's mass (at most 4.3e-8 over ~2800 draws of the
// configured workloads); normalised by the residual mass S that error grows
// by 1/S.  Down to S = kRefineMass of q_k's mass it stays below 7e-7, inside
// the 1e-6 window a draw's uniform must clear to be decided; a smaller
// residual (zero included) is refined: the draw is taken again in fp64 from
// the logits - both rows' normalisers, every tile's residual sum and the
// chosen tile's running sums - by the sequence's final item, in the single
// kernel or in the draw-and-final kernel where the kernels are separate.  In
// the bf16 single kernel that path needs more than its 64 registers and
// spills 92 bytes a lane to scratch, on that path only (no spill in the
// stream, sampling or draw code); a launch of its own would cost every call
// ~2-5 us.
constexpr double kRefineMass = 0.0625;           // refined below this fraction of q_k's mass
constexpr uint32_t kRefineToken = 0xFFFFFFFEu;   // drawn slot: the draw is refined (never a token id)
constexpr int kPendingWord = 8;                  // flag line: 1 = a refinement is pending

// e^x in fp64 for x <= 709 (0 below -745, and for -inf): x = n ln2 + r with
// |r| <= ln2 / 2, where ln2 is split into a 32-bit head (so n * head is exact)
// and its remainder; e^r by its Taylor polynomial of degree 12 (truncation
// below 3e-16 relative), scaled by 2^n.  Few registers, unlike the library
// routine, which matters inside the single kernel.
__device__ __forceinline__ double exp_f64(double x) {
  if (!(x > -745.0)) return 0.0;
  constexpr double kLog2e = 1.4426950408889634;
  constexpr double kLn2Hi = 0.6931471803691238;      // ln 2 with its low 21 significand bits clear
  constexpr double kLn2Lo = 1.9082149292705877e-10;  // ln 2 - kLn2Hi
  const double n = rint(x * kLog2e);
  const double r = fma(-n, kLn2Lo, fma(-n, kLn2Hi, x));
  double p = 1.0 / 479001600.0;   // 1/12!
  p = fma(p, r, 1.0 / 39916800.0);
  p = fma(p, r, 1.0 / 3628800.0);
  p = fma(p, r, 1.0 / 362880.0);
  p = fma(p, r, 1.0 / 40320.0);
  p = fma(p, r, 1.0 / 5040.0);
  p = fma(p, r, 1.0 / 720.0);
  p = fma(p, r, 1.0 / 120.0);
  p = fma(p, r, 1.0 / 24.0);
  p = fma(p, r, 1.0 / 6.0);
  p = fma(p, r, 0.5);
  p = fma(p, r, 1.0);
  p = fma(p, r, 1.0);
  return ldexp(p, (int)n);
}

// Logit pair j of rows k as fp64 exponentials relative to the references:
// et = exp(lt / T - mt), ed = exp(ld / T - md) (0 past the row, for a -inf
// logit, or one cut away by top-p).  Loaded on its own: this path is rare,
// and few live registers keep it from weighing on the single kernel.
template <int DT, bool CUT>
__device__ __forceinline__ void exp_pair(const void* drow, const void* trow, int64_t j, int64_t V, float Lt,
                                         float Ld, double invT, double mt, double md, double& et, double& ed) {
  float lt = -INFINITY, ld = -INFINITY;
  if (j < V) {
    lt = cut1<CUT>(load_one<DT>(trow, j), Lt);
    ld = cut1<CUT>(load_one<DT>(drow, j), Ld);
  }
  et = exp_f64(fma((double)lt, invT, -mt));
  ed = exp_f64(fma((double)ld, invT, -md));
}

// The drawn token of a sequence: the 64-bit word at byte 8 of its count line,
// stored as a complement (0 = not drawn yet).  kLostToken (never a token id)
// says that a wait of the draw gave up.
__device__ __forceinline__ uint64_t* drawn_slot(const VerifyArgs& a, int b) {
  return reinterpret_cast<uint64_t*>(SV_AT(a, flag, (int64_t)b * kFlagStride + 2));
}
constexpr uint32_t kLostToken = 0xFFFFFFFFu;

// The fp64 sums of tiles [t0, t1) of row pair k, each tile's four values in
// its refinement slots: E_t = sum et_j and E_d = sum ed_j over the tokens
// where et_j > ed_j, and the sums of et_j and ed_j over every token.  The
// references of the exponentials (Mt ln 2 for the target row; (Mt - K) ln 2
// for the draft row, log2(p_j / q_j) = (ld_j - lt_j) c_T + K) make et_j and
// ed_j equal q_j and p_j up to one common factor each, and those factors
// agree to the fp32 normalisers' precision, so the exact residual is
// (et_j - rho ed_j)+ / sum et with rho = sum et / sum ed = 1 + O(1e-7): a
// token whose et_j and ed_j agree to 2^-16 could fall on either side of the
// condition, and its tile is marked (E_t = NaN) to be summed again with the
// exact rho.
__device__ __forceinline__ uint64_t* ref_slots(const VerifyArgs& a, int b, int t) {
  return SV_AT(a, ref, ((int64_t)b * a.ntile + t) * 4);
}
struct RefineRefs {
  double invT, mt, md;
};
__device__ __forceinline__ RefineRefs refine_refs(const VerifyArgs& a, int b, const SeqRec& rec) {
  constexpr double kLn2 = 0.69314718055994530942;
  RefineRefs r;
  r.invT = temp_coef(a, b).invT;
  r.mt = (double)rec.Mt * kLn2;
  r.md = ((double)rec.Mt - ((double)rec.K_hi + (double)rec.K_lo)) * kLn2;
  return r;
}

struct RefineCtx {
  const void* drow;
  const void* trow;
  float Lt, Ld;
  double invT, mt, md;
};
template <int DT, bool CUT>
__device__ __forceinline__ RefineCtx refine_ctx(const VerifyArgs& a, int b, const SeqRec& rec) {
  RefineCtx c;
  draw_rows<DT>(a, b, rec.k, c.drow, c.trow);
  const SampleCoef cf = coef_of<CUT>(a, b, rec, 0.f);
  c.Lt = cf.Lt;
  c.Ld = cf.Ld;
  const RefineRefs rr = refine_refs(a, b, rec);
  c.invT = rr.invT;
  c.mt = rr.mt;
  c.md = rr.md;
  return c;
}

template <int DT, bool CUT>
__device__ __forceinline__ void refine_tiles(const VerifyArgs& a, int b, const SeqRec& rec, int t0, int t1,
                                             double* lds_d) {
  const RefineCtx c = refine_ctx<DT, CUT>(a, b, rec);
  for (int t = t0; t < t1; ++t) {
    double v[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    const int64_t j0 = (int64_t)t * kTile + (int64_t)threadIdx.x * kUnit;
#pragma unroll 1
    for (int e = 0; e < kUnit; ++e) {
      double et, ed;
      exp_pair<DT, CUT>(c.drow, c.trow, j0 + e, a.V, c.Lt, c.Ld, c.invT, c.mt, c.md, et, ed);
      v[2] += et;
      v[3] += ed;
      if (et > ed) {
        v[0] += et;
        v[1] += ed;
      }
      if (fabs(et - ed) <= 0x1p-16 * (et + ed) && et + ed > 0.0) v[4] = 1.0;
    }
    block_sum_n<5>(v, lds_d);
    if (threadIdx.x == 0) {
      uint64_t* r = ref_slots(a, b, t);
      slot_put(r + 0, v[4] > 0.0 ? __longlong_as_double(0x7FF8000000000000ll) : v[0]);
      slot_put(r + 1, v[1]);
      slot_put(r + 2, v[2]);
      slot_put(r + 3, v[3]);
    }
  }
}

// The refined draw of sequence b: sums every tile in fp64 (refine_tiles),
// forms rho from the exact sums, the tiles' residual sums (a marked tile
// again, with the exact rho), locates u * S in token order and rescans the
// tile in fp64: the oracle's residual ("Speculative Decoding: small model
// guesses, large model verifies", section 3, choice over (q - p)+ /
// sum (q - p)+).  A residual below 2^-40 of q_k's mass draws from q_k (the
// zero-mass reading).  Sets sh.y and the normalised S, pi(y), C_{y-1}, C_y;
// leaves the refinement and tile slots zero.
template <int DT, bool CUT>
__device__ __forceinline__ void refine_draw(const VerifyArgs& a, int b, const SeqRec& rec, DrawLds& sh) {
  const int tid = threadIdx.x, k = rec.k;
  refine_tiles<DT, CUT>(a, b, rec, 0, a.ntile, sh.lds_d);
  if (tid == 0) wait_mem();
  __syncthreads();
  uint64_t* tiles = SV_AT(a, tiles, (int64_t)b * a.ntile);
  // Normalisers (every thread sums its tiles, in tile order within the thread).
  double z[2] = {0.0, 0.0};
  for (int t = tid; t < a.ntile; t += kThreads) {
    uint64_t* r = ref_slots(a, b, t);
    z[0] += slot_value(poll(a, r + 2));
    z[1] += slot_value(poll(a, r + 3));
  }
  block_sum_n<2>(z, sh.lds_d);
  const double Zt = uni(z[0]), rho = uni(z[0] / z[1]);
  // Tile sums of the residual; marked tiles are counted and summed below.
  double tot = 0.0;
  int marked = 0;
  for (int t = tid; t < a.ntile; t += kThreads) {
    uint64_t* r = ref_slots(a, b, t);
    const double et = slot_value(poll(a, r + 0)), ed = slot_value(poll(a, r + 1));
    if (et != et) {
      ++marked;
    } else {
      const double w = fmax(et - rho * ed, 0.0);
      slot_put(tiles + t, w);
      tot += w;
    }
  }
  const RefineCtx c = refine_ctx<DT, CUT>(a, b, rec);
  const int64_t lane_off = (int64_t)tid * kUnit;
  if (block_min_int(-marked, sh.lds_i) < 0) {
    for (int t = 0; t < a.ntile; ++t) {
      const double et0 = slot_value(ld_dev_u64(ref_slots(a, b, t)));
      if (et0 == et0) continue;   // not marked
      double ws = 0.0;
#pragma unroll 1
      for (int e = 0; e < kUnit; ++e) {
        double et, ed;
        exp_pair<DT, CUT>(c.drow, c.trow, (int64_t)t * kTile + lane_off + e, a.V, c.Lt, c.Ld, c.invT, c.mt, c.md,
                          et, ed);
        ws += fmax(et - rho * ed, 0.0);
      }
      ws = block_sum(ws, sh.lds_d);
      if (tid == 0) slot_put(tiles + t, ws);
      if (tid == 0) tot += ws;
    }
  }
  tot = block_sum(tot, sh.lds_d);
  int mode = kModeResidual;
  if (!(tot > 0x1p-40 * Zt)) {   // a zero residual: draw from q_k
    mode = kModeTarget;
    for (int t = tid; t < a.ntile; t += kThreads) slot_put(tiles + t, slot_value(ld_dev_u64(ref_slots(a, b, t) + 2)));
  }
  wait_mem();
  __syncthreads();
  const double u = (double)*SV_AT(a, u_smp, ((int64_t)b * (a.gamma + 1) + k));
  double target;
  const double S = uni(locate_tile(tiles, a.ntile, u, sh, target));
  target = uni(target);
  // The chosen tile's running sums in fp64: every thread sums its unit; the
  // owner lane's unit is then walked by thread 0, one logit at a time.
  const int tsel = (int)SV_IDX(a, sh.tile, a.ntile);
  const int64_t jt = (int64_t)tsel * kTile;
  double ws = 0.0;
#pragma unroll 1
  for (int e = 0; e < kUnit; ++e) {
    double et, ed;
    exp_pair<DT, CUT>(c.drow, c.trow, jt + lane_off + e, a.V, c.Lt, c.Ld, c.invT, c.mt, c.md, et, ed);
    ws += mode == kModeResidual ? fmax(et - rho * ed, 0.0) : et;
  }
  double tile_tot;
  const double off = block_exclusive_scan(ws, sh.lds_d, tile_tot);
  const double tgt = target - sh.off;
  const int hit = (ws > 0.0 && off <= tgt && tgt < off + ws) ? tid : INT_MAX;
  int owner = block_min_int(hit, sh.lds_i);
  if (owner == INT_MAX) owner = -block_min_int(ws > 0.0 ? -tid : 1, sh.lds_i);   // last lane with weight
  if (tid == owner) sh.lane_off = off;
  __syncthreads();
  if (tid == 0) {
    double run = sh.lane_off, lo = run, lo_last = run;
    int idx = -1, last = -1;
    if (owner >= 0) {
#pragma unroll 1
      for (int e = 0; e < kUnit; ++e) {
        double et, ed;
        exp_pair<DT, CUT>(c.drow, c.trow, jt + (int64_t)owner * kUnit + e, a.V, c.Lt, c.Ld, c.invT, c.mt, c.md, et,
                          ed);
        const double we = mode == kModeResidual ? fmax(et - rho * ed, 0.0) : et;
        sh.w8d[e] = we;
        if (we > 0.0) {
          if (idx < 0 && tgt < run + we) {
            idx = e;
            lo = run;
          }
          last = e;
          lo_last = run;
        }
        run += we;
      }
    }
    if (idx < 0) {
      idx = last;
      lo = lo_last;
    }
    const double wy = idx >= 0 ? sh.w8d[idx] : 0.0;
    sh.y = idx >= 0 ? (int)((int64_t)tsel * kTile + (int64_t)owner * kUnit + idx)
                    : (int)min<int64_t>(a.V - 1, (int64_t)tsel * kTile + kTile - 1);   // not reached
    sh.n_rm = mode == kModeResidual ? S / Zt : 0.0;
    sh.n_tp = wy / S;
    sh.n_lo = (sh.off + lo) / S;
    sh.n_hi = (sh.off + lo + wy) / S;
  }
  __syncthreads();
  for (int t = tid; t < a.ntile; t += kThreads) {
    slot_clear(tiles + t);
    uint64_t* r = ref_slots(a, b, t);
#pragma unroll
    for (int i = 0; i < 4; ++i) slot_clear(r + i);
  }
}


// The draw at the stopping position: tile values, locate, rescan.  The token
// goes to the sequence's drawn slot, the diagnostics out.  Clears the tile and
// residual-sum slots once read.
template <int DT, bool VEC, bool CUT = false, bool EPS = true>
__device__ __forceinline__ void draw_item(const VerifyArgs& a, int b, DrawLds& sh) {
  const int tid = threadIdx.x;
  const SeqRec rec = wait_rec<true>(a, b);
  if (!rec.valid) return;
  const int g = a.gamma, k = rec.k;
  uint64_t* tiles = SV_AT(a, tiles, (int64_t)b * a.ntile);
  const float epsS = rec.mode == kModeSaguaroEps ? eps_clamp(a, b, sh.lds_d) : 0.f;
  const SampleCoef cf = coef_of<CUT>(a, b, rec, epsS);
  int mode = rec.mode;
  const double u = (double)*SV_AT(a, u_smp, ((int64_t)b * (g + 1) + k));   // in flight while the tiles arrive
  int lost = 0;   // a wait gave up: no token is drawn from what arrived
  uint64_t own = 0;   // tile tid's slot word as polled
  for (int t = tid; t < a.ntile; t += kThreads) {
    const uint64_t w = poll(a, tiles + t);
    if (t == tid) own = w;
    lost |= w == 0ull;
  }
  double rtot = 0.0;   // residual mass (relative to Mt) when it differs from the tile total
  if (mode == kModeSaguaro || mode == kModeSaguaroEps) {
#if SV_CHECKS
    uint64_t* rs = mode == kModeSaguaro ? SV_AT(a, rsum, (int64_t)b * a.nt) : SV_AT(a, mass, (int64_t)b * a.nt);
#else
    uint64_t* rs = (mode == kModeSaguaro ? a.rsum : a.mass) + (int64_t)b * a.nt;
#endif
    for (int i = tid; i < a.nt; i += kThreads) {
      const uint64_t w = poll(a, rs + i);
      lost |= w == 0ull;
      rtot += slot_value(w);
    }
  }
  rtot = uni(block_sum(rtot, sh.lds_d));   // also orders the polls before the reads below
  if (block_min_int(-lost, sh.lds_i) < 0 || (mode == kModeSaguaroEps && !(epsS == epsS))) {
    if (tid == 0) st_dev_u64(drawn_slot(a, b), ~(uint64_t)kLostToken);
    __syncthreads();
    for (int t = tid; t < a.ntile; t += kThreads) slot_clear(tiles + t);
    if (mode == kModeSaguaro)
      for (int i = tid; i < a.nt; i += kThreads) slot_clear(SV_AT(a, rsum, (int64_t)b * a.nt + i));
    if (mode == kModeSaguaroEps)
      for (int i = tid; i < a.nt; i += kThreads) slot_clear(SV_AT(a, mass, (int64_t)b * a.nt + i));
    return;
  }

  double target = 0.0, S = 0.0;
  if (tid == 0) sh.Mp = 0.0;
  // A zero Saguaro normaliser falls back to the residual; one pass per mode.
  // The Saguaro weights count as zero below 2^-21 of q_k's mass (rec.Zt, draw
  // units): where p_k and q_k agree, the fp32 weights leave only rounding (a
  // few ulp of q_k), below that.  A residual mass below kRefineMass of q_k's
  // (zero included: the draw from q_k) is refined in fp64.  A top-p cut can
  // make both rows the same one-token distribution; otherwise only degenerate
  // inputs get a zero residual.
  const double zero_res = 0x1p-21 * rec.Zt;
  const bool diag_req = a.diag.resid_mass || a.diag.token_prob || a.diag.cdf_lo || a.diag.cdf_hi;
  bool refine = false;
  // held: every tile value is in a register of its thread (at most kThreads
  // tiles, slots as polled), so the first scan reads no slot again.
  bool held = a.ntile <= kThreads;
  double hv = (held && tid < a.ntile) ? slot_value(own) : 0.0;
  if ((mode == kModeSaguaro || mode == kModeSaguaroEps) && rtot <= zero_res) {
    mode = kModeTarget;
    recompute_tiles<DT, CUT>(a, b, k, mode, cf, sh);
    held = false;   // the slots were rewritten
  }
  if (mode == kModeTarget && k == g) {   // the bonus draw: log2 tile values made linear
    if (held) {   // in registers, as tiles_to_linear does in the slots
      float m = tid < a.ntile ? (float)hv : -INFINITY;
      m = block_max(m, reinterpret_cast<float*>(sh.lds_d));
      const double Mp = isfinite(m) ? ceil((double)m) + 1.0 : 0.0;
      hv = (tid < a.ntile && hv > -INFINITY) ? exp2(hv - Mp) : 0.0;
      if (tid == 0) sh.Mp = Mp;
    } else {
      tiles_to_linear(tiles, a.ntile, sh);
    }
  }
  for (;;) {
    S = uni(held ? locate_tile_held(hv, a.ntile, u, sh, target) : locate_tile(tiles, a.ntile, u, sh, target));
    held = false;   // a second pass follows a rewrite of the slots
    target = uni(target);
    if (mode == kModeResidual) {
      rtot = S;
      if (S < kRefineMass * rec.Zt) {   // a small residual mass (zero included): refined
        refine = a.refine != 0;
        if (refine) break;
        if (S <= zero_res) S = 0.0;     // no refinement: a zero residual draws from q_k
      }
    }
    if (S > 0.0 || mode == kModeTarget) break;
    mode = mode == kModeResidual ? kModeTarget : kModeResidual;   // a zero Saguaro normaliser, or residual
    recompute_tiles<DT, CUT>(a, b, k, mode, cf, sh);
  }
  if (!refine) {
    with_mode<EPS>(mode, [&](auto m) { rescan_tile<DT, VEC, decltype(m)::value, CUT>(a, b, k, cf, target, sh); });
    if (diag_req && tid == 0) {
      sh.n_rm = k < g ? rtot / rec.Zt : 0.0;
      sh.n_tp = precise_weight<DT, CUT, EPS>(a, b, k, mode, cf, sh.y, sh) / S;
      sh.n_lo = sh.lo / S;
      sh.n_hi = sh.hi / S;
    }
  }
  if (tid == 0) {
    if (!refine) {
      if (a.diag.resid_mass) a.diag.resid_mass[SV_IDX(a, b, a.B)] = sh.n_rm;
      if (a.diag.token_prob) a.diag.token_prob[SV_IDX(a, b, a.B)] = sh.n_tp;
      if (a.diag.cdf_lo) a.diag.cdf_lo[SV_IDX(a, b, a.B)] = sh.n_lo;
      if (a.diag.cdf_hi) a.diag.cdf_hi[SV_IDX(a, b, a.B)] = sh.n_hi;
    }
    st_dev_u64(drawn_slot(a, b), ~(uint64_t)(refine ? kRefineToken : (uint32_t)sh.y));
  }
  // Every tile and residual-sum slot of the sequence has been read.
  __syncthreads();
  for (int t = tid; t < a.ntile; t += kThreads) slot_clear(tiles + t);
  if (rec.mode == kModeSaguaro)
    for (int i = tid; i < a.nt; i += kThreads) slot_clear(SV_AT(a, rsum, (int64_t)b * a.nt + i));
  if (rec.mode == kModeSaguaroEps)
    for (int i = tid; i < a.nt; i += kThreads) slot_clear(SV_AT(a, mass, (int64_t)b * a.nt + i));
}

// ---------------------------------------------------------------------------
// Final item: target row gamma, which only the bonus draw reads and which is
// therefore streamed last, is checked, and the outputs are written.

struct FinalLds {
  int ok, y, refine;
  DrawLds r;   // INLINE: the refined draw
};

template <int DT, bool CUT>
__device__ __forceinline__ void refine_item(const VerifyArgs& a, int b, DrawLds& sh);

// INLINE: a refined draw is taken here, by this work-group, after the
// outputs (in the single kernel its refined draws spill a few registers to
// scratch, on that path only); CUT: the rows are cut to their nuclei.
template <int DT, bool INLINE = false, bool CUT = false>
__device__ __forceinline__ void final_item(const VerifyArgs& a, int b, FinalLds& sh) {
  const int tid = threadIdx.x;
  const int g = a.gamma, R = 2 * g + 1, r = 2 * g;
  bool lost_rec;
  const SeqRec rec = wait_rec<false>(a, b, lost_rec);
  if (tid < 16) {
    double M, z;
    float mr;
    merge_row(a, b, r, tid, M, z, mr);
    if (tid == 0) {
      const bool ok = row_ok(M, z);
      sh.ok = ok;
      const bool read = !a.early || (rec.valid && rec.k == g);
      if (ok && read && a.diag.row_max)
        a.diag.row_max[SV_IDX(a, (int64_t)b * R + r, (int64_t)a.B * R)] = (double)mr * temp_coef(a, b).invT;
      if (ok && read && a.diag.row_logZ)
        a.diag.row_logZ[SV_IDX(a, (int64_t)b * R + r, (int64_t)a.B * R)] = M * 0.69314718055994530942 + log(z);
      sh.y = -1;
      sh.refine = 0;
      if (rec.valid) {
        uint64_t* ys = drawn_slot(a, b);
        const uint64_t w = poll(a, ys);
        const uint32_t y = (uint32_t)~w;
        sh.refine = w != 0ull && y == kRefineToken;
        sh.y = (w == 0ull || y == kLostToken || y == kRefineToken) ? -1 : (int)y;   // -1: lost (or refined below)
        slot_clear(ys);
      }
    }
  }
  __syncthreads();
  const bool refine = uni(sh.refine) != 0;   // the token at k comes from the refined draw
  if (lost_rec) {   // no decision arrived: nothing can be reported but an invalid sequence
    write_invalid(a, b, tid);
  } else if (rec.valid) {   // an invalid decision wrote its outputs already
    const int k = rec.k;
    if ((!sh.ok && (!a.early || k == g)) || (sh.y < 0 && !refine)) {   // early exit reads target row
      write_invalid(a, b, tid);   // gamma only for the bonus; sh.y < 0: the draw was lost
    } else {
      const int64_t orow = (int64_t)b * (g + 1);
      if (tid <= g) {
        int tok = -1;
        if (tid < k) tok = *SV_AT(a, tokens, ((int64_t)b * g + tid));
        else if (tid == k) tok = sh.y;
        *SV_AT(a, out_tokens, (orow + tid)) = tok;
      }
      if (tid == 0) {
        *SV_AT(a, out_acc, b) = k;
        if (a.out_first_reject) *SV_AT(a, out_first_reject, b) = k < g ? k : -1;
        if (a.out_mask) *SV_AT(a, out_mask, b) = rec.mask;
        if (a.out_len) *SV_AT(a, out_len, b) = (a.in_len ? *SV_AT(a, in_len, b) : 0) + k + 1;
      }
    }
  }
  // Once every other item of the sequence is done with the decision record,
  // clear it and the count.
  if (tid == 0) {
    unsigned* f = SV_AT(a, flag, (int64_t)b * kFlagStride);
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
    if (refine)   // refine_item reads the record, then clears it and the pending word
      __hip_atomic_store(f + kPendingWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      clear_rec(SV_AT(a, seq, b));
  }
  if constexpr (INLINE) {
    if (refine) {
      __syncthreads();
      refine_item<DT, CUT>(a, b, sh.r);
    }
  }
}

// ---------------------------------------------------------------------------
// Refinement: a refined residual draw (see kRefineMass), taken by the
// sequence's final item once its outputs are written; with no pending
// refinement it returns at once.
template <int DT, bool CUT>
__device__ __forceinline__ void refine_item(const VerifyArgs& a, int b, DrawLds& sh) {
  unsigned* f = SV_AT(a, flag, (int64_t)b * kFlagStride);
  if (ld_dev_u32(f + kPendingWord) == 0u) return;
  bool lost;
  const SeqRec rec = wait_rec<false>(a, b, lost);
  if (!lost && rec.valid && rec.k < a.gamma) {
    refine_draw<DT, CUT>(a, b, rec, sh);
    if (threadIdx.x == 0) {
      *SV_AT(a, out_tokens, ((int64_t)b * (a.gamma + 1) + rec.k)) = sh.y;
      if (a.diag.resid_mass) a.diag.resid_mass[SV_IDX(a, b, a.B)] = sh.n_rm;
      if (a.diag.token_prob) a.diag.token_prob[SV_IDX(a, b, a.B)] = sh.n_tp;
      if (a.diag.cdf_lo) a.diag.cdf_lo[SV_IDX(a, b, a.B)] = sh.n_lo;
      if (a.diag.cdf_hi) a.diag.cdf_hi[SV_IDX(a, b, a.B)] = sh.n_hi;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    clear_rec(SV_AT(a, seq, b));
    slot_clear32(f + kPendingWord);
  }
}

}  // namespace sv
