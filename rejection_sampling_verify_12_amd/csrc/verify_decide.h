// Decision items (whole sequence) and early-exit test items (one position).
#pragma once
#include "verify_stream.h"

#undef SV_FILE
#define SV_FILE 3

namespace sv {

// ---------------------------------------------------------------------------
// Decision of one sequence.

// Merge the chunk pieces of row r of sequence b within a 16-lane group (lane
// `sub` takes pieces sub, sub + 16, ...): M = the integer ceiling of
// max_c v_c, z = sum_c 2^(v_c - M) (fp64), mr = the row's largest raw logit.
// Waits for every piece (both words of a piece together) and clears them once
// read.  Every lane of the group returns the row's values.
__device__ __forceinline__ void merge_row(const VerifyArgs& a, int b, int r, int sub, double& M, double& z, float& mr) {
  const int64_t p0 = ((int64_t)b * (2 * a.gamma + 1) + r) * a.nc;
  M = -INFINITY;
  z = 0.0;
  mr = -INFINITY;
  double v0 = -INFINITY;   // the first piece stays in a register, later ones are read again
  for (int c = sub; c < a.nc; c += 16) {
    uint64_t wv = ld_dev_u64(SV_AT(a, part, p0 + c));
    unsigned wm = __hip_atomic_load(SV_AT(a, mraw, p0 + c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    unsigned polls = 0;
    while ((wv == 0ull || wm == 0u) && !give_up(a, polls)) {
      if (wv == 0ull) wv = ld_dev_u64(SV_AT(a, part, p0 + c));
      if (wm == 0u) wm = __hip_atomic_load(SV_AT(a, mraw, p0 + c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const double v = slot_value(wv);
    mr = fmaxf(mr, __uint_as_float(~wm));
    if (c == sub) v0 = v;
    M = fmax(M, v);
  }
#if SV_DPP
  M = row16_reduce(M, [](double x, double y) { return fmax(x, y); });
  mr = row16_reduce(mr, [](float x, float y) { return fmaxf(x, y); });
#else
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
    M = fmax(M, __shfl_xor(M, o, 16));
    mr = fmaxf(mr, __shfl_xor(mr, o, 16));
  }
#endif
  M = ceil(M);
  for (int c = sub; c < a.nc; c += 16) {
    const double v = c == sub ? v0 : slot_value(ld_dev_u64(SV_AT(a, part, p0 + c)));
    if (v != -INFINITY) z += exp2(v - M);   // a NaN piece stays NaN
    slot_clear(SV_AT(a, part, p0 + c));
    slot_clear32(SV_AT(a, mraw, p0 + c));
  }
#if SV_DPP
  z = row16_reduce(z, [](double x, double y) { return x + y; });
#else
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) z += __shfl_xor(z, o, 16);
#endif
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
  unsigned err;    // the error word, read with the gathers
};

// The rows the accept tests read, draft rows 0..gamma-1 and target rows
// 0..gamma-1 (16 lanes per row, 12 rows per pass), then the accept test at
// every draft position (wave 0, lane i = position i; fp64) and the decision
// record.  Target row gamma is checked by the sequence's final item.  A bad
// row or token makes the sequence invalid here, with its outputs.
template <int DT, bool CUT = false>
__device__ __forceinline__ void decide_item(const VerifyArgs& a, int b, DecideLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = a.gamma, Rd = 2 * g, R = 2 * g + 1;
  // Wave 1 gathers the draft tokens' logits and the uniforms (independent of
  // the row pieces) while waves 0, 2 and 3 merge the pieces.
  if (wave == 1) {
    if (lane < g) {
      const int x = *SV_AT(a, tokens, ((int64_t)b * g + lane));
      float ldx = 0.f, ltx = 0.f;
      if (x >= 0 && x < a.V) {
        ldx = load_one<DT>(row_ptr<DT>(a, b, lane), x);
        ltx = load_one<DT>(row_ptr<DT>(a, b, g + lane), x);
      }
      sh.x[lane] = x;
      sh.ldx[lane] = ldx;
      sh.ltx[lane] = ltx;
      sh.ux[lane] = *SV_AT(a, u_acc, ((int64_t)b * g + lane));
    }
    if (lane == 0) sh.err = ld_dev_u32(a.err);
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
    if (a.diag.row_max) a.diag.row_max[SV_IDX(a, (int64_t)b * R + r, (int64_t)a.B * R)] = (double)sh.mr[r] * tc.invT;
    if (a.diag.row_logZ)
      a.diag.row_logZ[SV_IDX(a, (int64_t)b * R + r, (int64_t)a.B * R)] = sh.M[r] * 0.69314718055994530942 + log(sh.Z[r]);
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
          const TopPRow* tpd = SV_AT(a, topp, (int64_t)b * R + lane);
          const TopPRow* tpt = SV_AT(a, topp, (int64_t)b * R + (g + lane));
          pn = sh.ldx[lane] >= tpd->L ? pn / tpd->P : 0.0;
          qn = sh.ltx[lane] >= tpt->L ? qn / tpt->P : 0.0;
        }
        double ratio;
        if (pn > 0.0) ratio = fmin(1.0, (qn * sh.Z[lane]) / (pn * sh.Z[g + lane]));
        else ratio = qn > 0.0 ? 1.0 : 0.0;
        acc = (double)sh.ux[lane] < ratio;
        if (a.diag.px) a.diag.px[SV_IDX(a, (int64_t)b * g + lane, (int64_t)a.B * g)] = pn / sh.Z[lane];
        if (a.diag.qx) a.diag.qx[SV_IDX(a, (int64_t)b * g + lane, (int64_t)a.B * g)] = qn / sh.Z[g + lane];
      }
    }
    const uint64_t mask = __ballot(acc);
    const uint64_t badm = __ballot(bad);
    if (lane == 0) {
      sh.mask = mask & ((1ull << g) - 1);
      // After a bounded wait has given up anywhere in the call (the error
      // word), a decision reports its sequence invalid.
      sh.valid = !rows_bad && badm == 0 && sh.err == 0u;
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
        Pt = SV_AT(a, topp, ((int64_t)b * R + g + k))->P;
        Pd = SV_AT(a, topp, ((int64_t)b * R + k))->P;
      }
      rec.Mt = (float)Mt;   // exact below 2^24; otherwise Zt absorbs the rounding
      rec.Zt = ldexp(sh.Z[g + k] * Pt, (int)fmin(fmax(Mt - (double)rec.Mt, -2000.0), 2000.0));
      const double K = (Mt - sh.M[k]) + log2((sh.Z[g + k] * Pt) / (sh.Z[k] * Pd));
      rec.K_hi = (float)K;
      rec.K_lo = (float)(K - (double)rec.K_hi);
    }
    store_rec(SV_AT(a, seq, b), rec);
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
  unsigned err;
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
__device__ __forceinline__ void test_item(const VerifyArgs& a, int b, int i, TestLds& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = a.gamma, R = 2 * g + 1;
  unsigned* fl = SV_AT(a, flag, (int64_t)b * kFlagStride);
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
    const int x = *SV_AT(a, tokens, ((int64_t)b * g + i));
    float ldx = 0.f, ltx = 0.f;
    if (x >= 0 && x < a.V) {
      ldx = load_one<DT>(row_ptr<DT>(a, b, i), x);
      ltx = load_one<DT>(row_ptr<DT>(a, b, g + i), x);
    }
    sh.x = x;
    sh.ldx = ldx;
    sh.ltx = ltx;
    sh.ux = *SV_AT(a, u_acc, ((int64_t)b * g + i));
    sh.err = ld_dev_u32(a.err);
  }
  __syncthreads();
  if (tid == 0) {
    const TCoef tc = temp_coef(a, b);
    const int x = sh.x;
    const bool bad = x < 0 || x >= a.V || sh.bad[0] || sh.bad[1] || (a.temps && !temp_ok(seq_temp(a, b))) ||
                     sh.err != 0u;   // a wait gave up somewhere: report the sequence invalid
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
      if (a.diag.px) a.diag.px[SV_IDX(a, (int64_t)b * g + i, (int64_t)a.B * g)] = pn / sh.Z[0];
      if (a.diag.qx) a.diag.qx[SV_IDX(a, (int64_t)b * g + i, (int64_t)a.B * g)] = qn / sh.Z[1];
      if (a.diag.row_max) {
        a.diag.row_max[SV_IDX(a, (int64_t)b * R + i, (int64_t)a.B * R)] = (double)sh.mr[0] * tc.invT;
        a.diag.row_max[SV_IDX(a, (int64_t)b * R + g + i, (int64_t)a.B * R)] = (double)sh.mr[1] * tc.invT;
      }
      if (a.diag.row_logZ) {
        a.diag.row_logZ[SV_IDX(a, (int64_t)b * R + i, (int64_t)a.B * R)] =
            sh.M[0] * 0.69314718055994530942 + log(sh.Z[0]);
        a.diag.row_logZ[SV_IDX(a, (int64_t)b * R + g + i, (int64_t)a.B * R)] =
            sh.M[1] * 0.69314718055994530942 + log(sh.Z[1]);
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
    store_rec(SV_AT(a, seq, b), rec);
  }
}

}  // namespace sv
