// Outcome prediction for speculative speculative decoding on gfx950.
//
// "Speculative Speculative Decoding (Saguaro)", section 3.1: a verification
// outcome is (k accepted, bonus token); the bonus is predicted from the draft
// logits' top-3.  For every sequence and every k in 0..gamma the three
// largest draft logits at position k are the candidates for the token emitted
// after k acceptances; after the real verification, hit = the emitted token is
// among the candidates of the realised k.
//
// Kernel 1 (top3_chunk): one work-group per (sequence, position, chunk)
//   streams a chunk of a draft row (16-byte nontemporal loads) and keeps each
//   lane's best three (value, index), testing eight elements at a time on
//   their maximum; the lanes' candidates become 64-bit keys (order-preserving
//   map of the logit's bits, then the complemented token id so that equal
//   logits rank the lower id first) and three rounds of a work-group max
//   extract the chunk's top-3.
// Kernel 2 (top3_merge): one wave per sequence merges the chunk candidates of
//   each position and evaluates the hit.
#include "common.h"
#include "spec_verify.h"

#include <limits.h>

namespace sv {

struct Top3 {
  uint64_t key[3];
  uint64_t nan;   // nonzero when the chunk held a NaN
};

// Order-preserving key: larger logit -> larger key; equal logits -> lower id
// larger.  -0.0 is folded onto +0.0.  0 never occurs for a real element.
__device__ __forceinline__ uint64_t make_key(uint32_t bits, int64_t idx) {
  if (bits == 0x80000000u) bits = 0u;
  const uint32_t mono = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  return ((uint64_t)mono << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
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

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* lds) {
  v = wave_max_u64(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) lds[w] = v;
  __syncthreads();
  uint64_t t = lds[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) t = lds[i] > t ? lds[i] : t;
  __syncthreads();
  return t;
}

struct PredictArgs {
  const void* draft;
  const int32_t* accepted;
  const int32_t* out_tokens;
  int32_t* cand;
  int32_t* hit;
  int32_t* cand_idx;
  Top3* part;   // [B][gamma+1][nc]
  int B, gamma, V, nc;
};

// A lane's best three elements, largest first.  Elements arrive in increasing
// index order, so an equal value never displaces an earlier one (ties go to
// the lower id); an empty slot holds (-inf, INT_MAX) and takes any non-NaN
// value.  +0.0 and -0.0 compare equal.  A NaN never enters.
struct Best3 {
  float v[3];
  int i[3];
};

__device__ __forceinline__ bool beats(float v, float sv, int si) {
  return v > sv || (v == sv && si == INT_MAX);
}

__device__ __forceinline__ void offer(Best3& t, float v, int idx) {
  if (!beats(v, t.v[2], t.i[2])) return;
  if (beats(v, t.v[1], t.i[1])) {
    t.v[2] = t.v[1];
    t.i[2] = t.i[1];
    if (beats(v, t.v[0], t.i[0])) {
      t.v[1] = t.v[0];
      t.i[1] = t.i[0];
      t.v[0] = v;
      t.i[0] = idx;
    } else {
      t.v[1] = v;
      t.i[1] = idx;
    }
  } else {
    t.v[2] = v;
    t.i[2] = idx;
  }
}

// Eight elements of a lane (indices j0..j0+7, those < end): a cheap test on
// their maximum first, the careful insertion only when it can change the best
// three; NaN bits are or-ed into `nan`.
template <int DT, bool VEC>
__device__ __forceinline__ void offer8(Best3& t, const Raw8<DT, VEC>& raw, int64_t j0, int64_t end,
                                       bool full, uint32_t& nan) {
  float v[8];
  unpack<DT, VEC>(raw, v);
  if constexpr (DT == kBF16 && VEC) {   // (h & 0x7FFF) > 0x7F80 per half: a NaN
    const uint32_t w[4] = {raw.w.x, raw.w.y, raw.w.z, raw.w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) nan |= ((w[q] & 0x7FFF7FFFu) + 0x007F007Fu) & 0x80008000u;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) nan |= (uint32_t)(v[e] != v[e]);
  }
  float m = v[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) m = fmaxf(m, v[e]);
  if (!full || beats(m, t.v[2], t.i[2])) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (full || j0 + e < end) offer(t, v[e], (int)(j0 + e));
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void top3_chunk_kernel(PredictArgs a) {
  __shared__ uint64_t lds[kWaves];
  __shared__ int lds_i[kWaves];
  const int64_t id = blockIdx.x;
  const int64_t row = id / a.nc;   // b * (gamma+1) + k
  const int c = (int)(id - row * a.nc);
  constexpr int kEs = DT == kBF16 ? 2 : 4;
  const void* rp = static_cast<const char*>(a.draft) + row * (int64_t)a.V * kEs;
  const int64_t begin = (int64_t)c * kChunk;
  const int64_t end = min<int64_t>(begin + kChunk, a.V);
  constexpr int U = 4;
  constexpr int64_t kStep = (int64_t)kThreads * kUnit, kBatch = U * kStep;
  Best3 t;
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    t.v[r] = -INFINITY;
    t.i[r] = INT_MAX;
  }
  uint32_t nan = 0;
  int64_t j;
  if constexpr (VEC) {
    // Full batches through a buffer resource over the chunk (nontemporal).
    const int nb = (int)((end - begin) / kBatch);
    const __amdgpu_buffer_rsrc_t rs =
        chunk_rsrc(static_cast<const char*>(rp) + begin * kEs, (int)((end - begin) * kEs));
    const int voff = (int)threadIdx.x * kUnit * kEs;
    for (int i = 0; i < nb; ++i) {
      Raw8<DT, VEC> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) load_raw_buf<DT>(rs, voff, (int)((i * kBatch + u * kStep) * kEs), raw[u]);
#pragma unroll
      for (int u = 0; u < U; ++u)
        offer8<DT, VEC>(t, raw[u], begin + i * kBatch + u * kStep + (int64_t)threadIdx.x * kUnit, end, true, nan);
    }
    j = begin + nb * kBatch + (int64_t)threadIdx.x * kUnit;
  } else {
    j = begin + (int64_t)threadIdx.x * kUnit;
  }
  for (; j < end; j += kStep) {   // the rest, unit by unit, bounds-checked
    Raw8<DT, VEC> raw;
    load_raw<DT, VEC, true>(rp, j, end, raw);
    offer8<DT, VEC>(t, raw, j, end, false, nan);
  }
  const int any_nan = -block_min_int(nan != 0 ? -1 : 0, lds_i);
  uint64_t k3[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) k3[r] = t.i[r] == INT_MAX ? 0 : make_key(__float_as_uint(t.v[r]), t.i[r]);
  uint64_t best[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    best[r] = block_max_u64(k3[0], lds);
    if (best[r] != 0 && k3[0] == best[r]) {   // keys are unique: the owner pops it
      k3[0] = k3[1];
      k3[1] = k3[2];
      k3[2] = 0;
    }
  }
  if (threadIdx.x == 0) {
    Top3 o;
    o.key[0] = best[0];
    o.key[1] = best[1];
    o.key[2] = best[2];
    o.nan = (uint64_t)any_nan;
    a.part[id] = o;
  }
}

__global__ __launch_bounds__(64) void top3_merge_kernel(PredictArgs a) {
  __shared__ int s_cand[64 * 3];
  const int b = blockIdx.x;
  const int k = threadIdx.x;
  const int G1 = a.gamma + 1;
  if (k < G1) {
    const Top3* P = a.part + ((int64_t)b * G1 + k) * a.nc;
    uint64_t t[3] = {0, 0, 0};
    uint64_t nan = 0;
    for (int c = 0; c < a.nc; ++c) {
      nan |= P[c].nan;
#pragma unroll
      for (int r = 0; r < 3; ++r) insert3(t, P[c].key[r]);
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int tok = (nan || t[r] == 0) ? -1 : (int)(0xFFFFFFFFu - (uint32_t)(t[r] & 0xFFFFFFFFu));
      s_cand[k * 3 + r] = tok;
      a.cand[((int64_t)b * G1 + k) * 3 + r] = tok;
    }
  }
  __syncthreads();
  if (k == 0 && a.accepted && a.out_tokens) {
    const int K = a.accepted[b];
    int h = 0, idx = -1;
    if (K >= 0 && K < G1) {
      const int y = a.out_tokens[(int64_t)b * G1 + K];
      for (int r = 0; r < 3; ++r) {
        if (y >= 0 && s_cand[K * 3 + r] == y) {
          h = 1;
          idx = 3 * K + r;
          break;
        }
      }
    }
    if (a.hit) a.hit[b] = h;
    if (a.cand_idx) a.cand_idx[b] = idx;
  }
}

static inline size_t predict_bytes(int B, int gamma, int V) {
  if (B == 0) return 0;
  const size_t nc = (size_t)((V + kChunk - 1) / kChunk);
  return (((size_t)B * (gamma + 1) * nc * sizeof(Top3)) + 255) & ~(size_t)255;
}

}  // namespace sv

extern "C" {

size_t spec_predict_workspace_bytes(int B, int gamma, int V, int dtype) {
  if ((dtype != SPEC_F32 && dtype != SPEC_BF16) || B < 0 || gamma < 1 || gamma > 63 || V < 1)
    return 0;
  return sv::predict_bytes(B, gamma, V);
}

int spec_predict_outcomes(const void* draft_logits, int dtype, int B, int gamma, int V,
                          const int32_t* accepted, const int32_t* out_tokens, int32_t* cand,
                          int32_t* hit, int32_t* cand_idx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  using namespace sv;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (B < 0 || gamma < 1 || gamma > 63 || V < 1) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!draft_logits || !cand) return SPEC_EINVAL;
  if ((accepted == nullptr) != (out_tokens == nullptr)) return SPEC_EINVAL;
  const int nc = (V + kChunk - 1) / kChunk;
  const int64_t nblk = (int64_t)B * (gamma + 1) * nc;
  if (nblk * kThreads > (int64_t)UINT_MAX) return SPEC_EINVAL;
  if (!workspace || workspace_bytes < predict_bytes(B, gamma, V)) return SPEC_EWORKSPACE;
  PredictArgs a;
  a.draft = draft_logits;
  a.accepted = accepted;
  a.out_tokens = out_tokens;
  a.cand = cand;
  a.hit = hit;
  a.cand_idx = cand_idx;
  a.part = static_cast<Top3*>(workspace);
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.nc = nc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool vec = (V % 8 == 0) && ((uintptr_t)draft_logits % 16 == 0);
  if (dtype == SPEC_BF16) {
    if (vec) hipLaunchKernelGGL((top3_chunk_kernel<kBF16, true>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((top3_chunk_kernel<kBF16, false>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((top3_chunk_kernel<kF32, true>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((top3_chunk_kernel<kF32, false>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
  }
  hipLaunchKernelGGL(top3_merge_kernel, dim3((unsigned)B), dim3(64), 0, st, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

}  // extern "C"
