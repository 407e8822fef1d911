// Stream items: one chunk of one row to its normaliser piece.
#pragma once
#include "verify_args.h"

#undef SV_FILE
#define SV_FILE 2

namespace sv {

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
  c = (int)SV_IDX(a, c, a.nc);
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
  // Through LDS lane permutes: with the DPP reductions here the early-exit
  // order's single kernel measured 176 against 159 us at B=256 (and the
  // default order no faster).
  const float wm = wave_max_lds(mref);
  const float wr = wave_max_lds(mraw);
  double sd = (s != 0.0) ? ldexp(s, (int)fmaxf(mref - wm, -2000.f)) : 0.0;
  sd = wave_sum_lds(sd);
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
    slot_put32(SV_AT(a, mraw, idx), mr);
    slot_put(SV_AT(a, part, idx), v);
    if constexpr (LEAD) store_leaders(sh, v != v, SV_AT(a, cpart, ((int64_t)b * (a.gamma + 1) + r) * a.nc + c));
  }
}

// Draft row gamma (outcome prediction only): one chunk's lane leaders and
// NaN flag, nothing else.
template <int DT, bool VEC, int U>
__device__ __forceinline__ void leader_item(const VerifyArgs& a, int b, int c, StreamLds& sh) {
  constexpr int kEs = DT == kBF16 ? 2 : 4;
#if SV_CHECKS
  b = (int)SV_IDX(a, b, a.B);
  c = (int)SV_IDX(a, c, a.nc);
#endif
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
    store_leaders(sh, any != 0, SV_AT(a, cpart, ridx * a.nc + c));
  }
}

// The outputs of an invalid sequence (threads 0..gamma).
__device__ __forceinline__ void write_invalid(const VerifyArgs& a, int b, int tid) {
  const int g = a.gamma;
  if (tid <= g) *SV_AT(a, out_tokens, ((int64_t)b * (g + 1) + tid)) = -1;
  if (tid == 0) {
    *SV_AT(a, out_acc, b) = -1;
    if (a.out_first_reject) *SV_AT(a, out_first_reject, b) = -1;
    if (a.out_mask) *SV_AT(a, out_mask, b) = 0;
    if (a.out_len) *SV_AT(a, out_len, b) = a.in_len ? *SV_AT(a, in_len, b) : 0;
  }
}

}  // namespace sv
