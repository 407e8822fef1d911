// Outcome prediction for speculative speculative decoding on gfx950.
//
// "Speculative Speculative Decoding (Saguaro)", section 3.1: a verification
// outcome is (k accepted, bonus token); the bonus is predicted from the draft
// logits' top-3.  For every sequence and every k in 0..gamma the three
// largest draft logits at position k are the candidates for the token emitted
// after k acceptances; after the real verification, hit = the emitted token is
// among the candidates of the realised k.
//
// Stand-alone path (spec_predict_outcomes):
// Kernel 1 (top3_chunk): one work-group per (sequence, position, chunk)
//   streams a chunk of a draft row (16-byte nontemporal loads) and keeps each
//   lane's best three (value, index), testing eight elements at a time on
//   their maximum; each wave extracts its top-3 keys and the first thread
//   merges the waves'.
// Kernel 2 (top3_merge): one wave per sequence merges the chunk candidates of
//   each position and evaluates the hit.
// Fused path (spec_verify_predict): the verification's stream items record
// each chunk's three best lane leaders (see topk.h); top3_lanes then re-reads
// the (at most three) leading lanes of every draft row, ranks their elements
// and evaluates the hit.
#include "common.h"
#include "predict.h"
#include "spec_verify.h"
#include "topk.h"

#include <limits.h>

namespace sv {

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

template <int DT>
__device__ __forceinline__ uint32_t load_bits(const void* row, int64_t j) {
  if constexpr (DT == kBF16) return (uint32_t)static_cast<const uint16_t*>(row)[j] << 16;
  else return static_cast<const uint32_t*>(row)[j];
}

// The work-group's three best keys and NaN flag from each wave's: the first
// lane of every wave leaves its wave's in LDS, thread 0 merges them.
struct ChunkLds {
  uint64_t key[kWaves * 3];
  int nan[kWaves];
};
__device__ __forceinline__ void chunk_top3(uint64_t (&t)[3], bool nan, ChunkLds& sh, Top3* out) {
  uint64_t w3[3];
  wave_top3(t, w3);
  const bool wn = __ballot(nan) != 0;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int r = 0; r < 3; ++r) sh.key[w * 3 + r] = w3[r];
    sh.nan[w] = wn ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t m[3] = {0, 0, 0};
    int any = 0;
    for (int i = 0; i < kWaves; ++i) {
      any |= sh.nan[i];
#pragma unroll
      for (int r = 0; r < 3; ++r) insert3(m, sh.key[i * 3 + r]);
    }
    Top3 o;
    o.key[0] = m[0];
    o.key[1] = m[1];
    o.key[2] = m[2];
    o.nan = (uint64_t)any;
    *out = o;
  }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void top3_chunk_kernel(PredictArgs a) {
  __shared__ ChunkLds sh;
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
  uint64_t k3[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) k3[r] = t.i[r] == INT_MAX ? 0 : make_key(__float_as_uint(t.v[r]), t.i[r]);
  chunk_top3(k3, nan != 0, sh, a.part + id);
}

// Hit flag and candidate index of sequence b from its candidates in LDS.
__device__ __forceinline__ void eval_hit(const PredictArgs& a, int b, const int* s_cand) {
  if (!a.accepted || !a.out_tokens) return;
  const int G1 = a.gamma + 1;
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
      const int tok = (nan || t[r] == 0) ? -1 : key_index(t[r]);
      s_cand[k * 3 + r] = tok;
      a.cand[((int64_t)b * G1 + k) * 3 + r] = tok;
    }
  }
  __syncthreads();
  if (k == 0) eval_hit(a, b, s_cand);
}

// One wave per (sequence, position).  The chunk records hold lane leaders
// (key index = start of the leader's best unit); the row's three best leaders
// are found first, then lanes 16l..16l+15 re-read leader l's units (every
// kTile-th unit of its chunk) and the wave ranks those elements.  The wave of
// the realised position (position 0 for an invalid sequence) also evaluates
// the hit; its emitted token is loaded while the leaders are re-read.
template <int DT>
__global__ __launch_bounds__(64) void top3_lanes_kernel(PredictArgs a) {
  const int G1 = a.gamma + 1;
  const int64_t row = blockIdx.x;   // b * (gamma + 1) + k
  const int b = (int)(row / G1), k = (int)(row - (int64_t)b * G1);
  const int lane = threadIdx.x;
  constexpr int kEs = DT == kBF16 ? 2 : 4;
  const bool with_hit = a.accepted && a.out_tokens;
  const int K = with_hit ? a.accepted[b] : -1;
  const bool mine_hit = with_hit && (K == k || ((K < 0 || K >= G1) && k == 0));
  const Top3* P = a.part + row * a.nc;
  // Lane l merges the records of chunks l, l + 64, ...; then the wave merges
  // the lanes.
  uint64_t t[3] = {0, 0, 0};
  bool nan_l = false;
  for (int c = lane; c < a.nc; c += 64) {
    const Top3 r = P[c];
    insert3(t, r.key[0]);
    insert3(t, r.key[1]);
    insert3(t, r.key[2]);
    nan_l = nan_l || r.nan != 0u;
  }
  const bool nan = __ballot(nan_l) != 0;
  uint64_t lead[3];
  wave_top3(t, lead);
  int y = -1;
  if (mine_hit && K == k) y = a.out_tokens[row];   // in flight with the re-read below
  const int l = lane >> 4;
  const uint64_t mine = l == 0 ? lead[0] : (l == 1 ? lead[1] : (l == 2 ? lead[2] : 0ull));
  uint64_t e3[3] = {0, 0, 0};
  if (mine != 0) {
    const void* rp = static_cast<const char*>(a.draft) + row * (int64_t)a.V * kEs;
    const int64_t s0 = key_index(mine);
    const int64_t cb = s0 / a.chunk * a.chunk;
    const int64_t ce = min<int64_t>(cb + a.chunk, a.V);
    for (int64_t j = s0 - (s0 - cb) / kTile * kTile + (int64_t)(lane & 15) * kTile; j < ce; j += 16 * kTile)
      for (int e = 0; e < kUnit && j + e < ce; ++e)
        insert3(e3, make_key(load_bits<DT>(rp, j + e), j + e));
  }
  uint64_t best[3];
  wave_top3(e3, best);
  int tok[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) tok[r] = (nan || best[r] == 0) ? -1 : key_index(best[r]);
  if (lane < 3) a.cand[row * 3 + lane] = lane == 0 ? tok[0] : (lane == 1 ? tok[1] : tok[2]);
  if (mine_hit && lane == 0) {
    int h = 0, idx = -1;
    if (K == k && y >= 0) {
#pragma unroll
      for (int r = 2; r >= 0; --r)
        if (tok[r] == y) {
          h = 1;
          idx = 3 * k + r;
        }
    }
    if (a.hit) a.hit[b] = h;
    if (a.cand_idx) a.cand_idx[b] = idx;
  }
}

size_t predict_part_bytes(int B, int gamma, int V) {
  if (B == 0) return 0;
  const size_t nc = (size_t)((V + kChunk - 1) / kChunk);
  return (((size_t)B * (gamma + 1) * nc * sizeof(Top3)) + 255) & ~(size_t)255;
}

hipError_t predict_launch_rows(const PredictArgs& a, int dtype, bool vec, hipStream_t st) {
  const int64_t nblk = (int64_t)a.B * (a.gamma + 1) * a.nc;
  if (dtype == SPEC_BF16) {
    if (vec) hipLaunchKernelGGL((top3_chunk_kernel<kBF16, true>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((top3_chunk_kernel<kBF16, false>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((top3_chunk_kernel<kF32, true>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((top3_chunk_kernel<kF32, false>), dim3((unsigned)nblk), dim3(kThreads), 0, st, a);
  }
  hipLaunchKernelGGL(top3_merge_kernel, dim3((unsigned)a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t predict_launch_leaders(const PredictArgs& a, int dtype, hipStream_t st) {
  const unsigned rows = (unsigned)((int64_t)a.B * (a.gamma + 1));
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL((top3_lanes_kernel<kBF16>), dim3(rows), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((top3_lanes_kernel<kF32>), dim3(rows), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv

extern "C" {

size_t spec_predict_workspace_bytes(int B, int gamma, int V, int dtype) {
  if ((dtype != SPEC_F32 && dtype != SPEC_BF16) || !sv::sizes_in_range(B, gamma, V))
    return 0;
  return sv::predict_part_bytes(B, gamma, V);
}

int spec_predict_outcomes(const void* draft_logits, int dtype, int B, int gamma, int V,
                          const int32_t* accepted, const int32_t* out_tokens, int32_t* cand,
                          int32_t* hit, int32_t* cand_idx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  using namespace sv;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (!sizes_in_range(B, gamma, V)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!draft_logits || !cand) return SPEC_EINVAL;
  if ((accepted == nullptr) != (out_tokens == nullptr)) return SPEC_EINVAL;
  const int nc = (V + kChunk - 1) / kChunk;
  const int64_t nblk = (int64_t)B * (gamma + 1) * nc;
  if (nblk * kThreads > (int64_t)UINT_MAX) return SPEC_EINVAL;
  if (!workspace || workspace_bytes < predict_part_bytes(B, gamma, V)) return SPEC_EWORKSPACE;
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
  a.chunk = kChunk;
  (void)hipGetLastError();
  const bool vec = (V % 8 == 0) && ((uintptr_t)draft_logits % 16 == 0);
  const hipError_t e = predict_launch_rows(a, dtype, vec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

}  // extern "C"
