// A timed stand-in for a model forward pass, for pipeline experiments around
// the verification ("Speculative Speculative Decoding (Saguaro)", section 4.1:
// the draft model runs on its own stream (and device) while the target
// verifies; SSD summary, AMD MI300X part: draft and target on separate HIP
// streams synchronised by events).  No model weights exist here, so a "model"
// is a kernel that keeps one work-group busy for a set wall time: it occupies
// its stream for that long without taking the compute units the verification
// uses, as a model on a separate device would.
#include "spec_verify.h"

#include "common.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sv {
namespace {

constexpr int64_t kMaxBusyNs = 100000000;   // 0.1 s

// s_memrealtime counts at 100 MHz on gfx950.  The loop ends after `ticks` of
// them (a bounded wait); with `hit`, it first checks whether any of the n
// flags is 0 and returns at once if none is (a speculation that hit needs no
// fallback pass).
__global__ __launch_bounds__(64) void busy_kernel(int64_t ticks, const int32_t* hit, int n) {
  __shared__ int any_miss;
  if (hit) {
    int miss = 0;
    for (int i = threadIdx.x; i < n; i += 64) miss |= hit[i] == 0;
    miss = __ballot(miss) != 0;
    if (threadIdx.x == 0) any_miss = miss;
    __syncthreads();
    if (!any_miss) return;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) < ticks) __builtin_amdgcn_s_sleep(8);
}

}  // namespace
}  // namespace sv

extern "C" int spec_synthetic_busy(int64_t ns, const int32_t* hit, int n, void* stream) {
  if (ns < 0 || ns > sv::kMaxBusyNs || n < 0 || (n > 0 && !hit)) return SPEC_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(sv::busy_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     (int64_t)((ns + 9) / 10), n > 0 ? hit : nullptr, n);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

// ---------------------------------------------------------------------------
// Synthetic bigram models and the pre-speculation of the next round.
//
// A bigram "model" gives, after token t, the logits of row t mod H of an
// [H][V] table (H = V: one row per token).  Its draft sampling is the Gumbel-max form: the token drawn at
// absolute position pos is argmax_j (table[t][j] + noise[pos mod P][j]),
// one fp32 addition per candidate and ties to the lower id, where noise holds
// T-scaled Gumbel variates (argmax of l/T + g draws from softmax(l/T)).
//
// "Speculative Speculative Decoding (Saguaro)", sections 3.1 and 4.1: while
// the target verifies round r, the draft prepares the next round's drafts for
// each outcome it predicts - k accepted tokens followed by one of the draft's
// top-3 tokens at position k - and a round whose outcome was among them starts
// from the prepared drafts; any other outcome drafts after the verification.

namespace sv {
namespace {

constexpr int kChainThreads = 1024;   // one work-group per chain: 16 waves of loads in flight
constexpr int kRowThreads = 256;
constexpr int kRowChunk = 16384;      // elements of a row per work-group of the row gather

template <int DT>
__device__ __forceinline__ float table_at(const void* t, size_t i) {
  if constexpr (DT == SPEC_BF16) {
    return __uint_as_float((uint32_t)(static_cast<const uint16_t*>(t)[i]) << 16);
  } else {
    return static_cast<const float*>(t)[i];
  }
}

// A key whose unsigned order is (score, then lower id): the float's bits made
// monotone in the upper half, the complemented id in the lower.  -0 takes the
// key of +0, so equal scores tie whatever their sign.
__device__ __forceinline__ uint64_t argmax_key(float s, int j) {
  s = s == 0.0f ? 0.0f : s;
  uint32_t u = __float_as_uint(s);
  u ^= (u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;
  return ((uint64_t)u << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}

__device__ __forceinline__ void keep_max(uint64_t& best, float s, int j) {
  const uint64_t k = argmax_key(s, j);
  best = k > best ? k : best;
}

// This thread's best key over one row: 16-byte loads (8 bf16 or 4 float logits
// and 4 noise values each) when the rows allow them, single elements otherwise.
template <int DT>
__device__ __forceinline__ uint64_t row_best(const void* table, size_t row, const float* g, int V,
                                             bool vec) {
  uint64_t best = 0;
  constexpr int W = DT == SPEC_BF16 ? 8 : 4;
  if (vec) {
    const int nv = V / W;
    for (int v = threadIdx.x; v < nv; v += kChainThreads) {
      const int j0 = v * W;
      const float4* gn = reinterpret_cast<const float4*>(g + j0);
      if constexpr (DT == SPEC_BF16) {
        const uint4 t = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(table) + row)[v];
        const float4 n0 = gn[0], n1 = gn[1];
        keep_max(best, __uint_as_float(t.x << 16) + n0.x, j0 + 0);
        keep_max(best, __uint_as_float(t.x & 0xFFFF0000u) + n0.y, j0 + 1);
        keep_max(best, __uint_as_float(t.y << 16) + n0.z, j0 + 2);
        keep_max(best, __uint_as_float(t.y & 0xFFFF0000u) + n0.w, j0 + 3);
        keep_max(best, __uint_as_float(t.z << 16) + n1.x, j0 + 4);
        keep_max(best, __uint_as_float(t.z & 0xFFFF0000u) + n1.y, j0 + 5);
        keep_max(best, __uint_as_float(t.w << 16) + n1.z, j0 + 6);
        keep_max(best, __uint_as_float(t.w & 0xFFFF0000u) + n1.w, j0 + 7);
      } else {
        const float4 t = reinterpret_cast<const float4*>(static_cast<const float*>(table) + row)[v];
        const float4 n0 = gn[0];
        keep_max(best, t.x + n0.x, j0 + 0);
        keep_max(best, t.y + n0.y, j0 + 1);
        keep_max(best, t.z + n0.z, j0 + 2);
        keep_max(best, t.w + n0.w, j0 + 3);
      }
    }
  } else {
    for (int j = threadIdx.x; j < V; j += kChainThreads) keep_max(best, table_at<DT>(table, row + j) + g[j], j);
  }
  return best;
}

// gamma draft steps of one work-group from token `tok` at position `pos`:
// out[i] is the token drawn at position pos + i.  A start token outside
// [0, V) gives -1 at every step.
template <int DT>
__device__ void draft_chain(const void* table, int V, int H, const float* noise, int P, int gamma,
                            int tok, int pos, int32_t* out) {
  __shared__ uint64_t red[kChainThreads / 64];
  __shared__ int bcast;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int W = DT == SPEC_BF16 ? 8 : 4;
  // every row and noise row starts on a 16-byte boundary when V is a multiple
  // of W (and of 4 for the noise) and both arrays do
  const bool vec = V % W == 0 && V % 4 == 0 &&
                   (((uintptr_t)table | (uintptr_t)noise) & 15) == 0;
  for (int i = 0; i < gamma; ++i) {
    if (tok < 0 || tok >= V) {   // the same for the whole work-group
      if (threadIdx.x == 0) out[i] = -1;
      continue;
    }
    const size_t row = (size_t)((unsigned)tok % (unsigned)H) * (size_t)V;
    const float* g = noise + (size_t)(((unsigned)pos + (unsigned)i) % (unsigned)P) * (size_t)V;
    uint64_t best = row_best<DT>(table, row, g, V, vec);
    for (int off = 32; off > 0; off >>= 1) {
      const uint64_t o = __shfl_xor((unsigned long long)best, off);
      best = o > best ? o : best;
    }
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t b = red[0];
      for (int w = 1; w < kChainThreads / 64; ++w) b = red[w] > b ? red[w] : b;
      tok = (int)(0xFFFFFFFFu - (uint32_t)b);
      out[i] = tok;
      bcast = tok;
    }
    __syncthreads();
    tok = bcast;
  }
}

template <int DT>
__global__ __launch_bounds__(kChainThreads) void draft_kernel(
    const void* table, int V, int H, const float* noise, int P, int gamma, const int32_t* start_tok,
    const int32_t* start_pos, int32_t* out) {
  const int c = blockIdx.x;
  draft_chain<DT>(table, V, H, noise, P, gamma, start_tok[c], start_pos ? start_pos[c] : 0,
                  out + (size_t)c * gamma);
}

// One work-group per (sequence b, candidate c = 3k + rank): the drafts that
// follow outcome "k accepted, then cand[b][k][rank]", from position len[b] + k + 1.
template <int DT>
__global__ __launch_bounds__(kChainThreads) void prespec_kernel(
    const void* table, int V, int H, const float* noise, int P, int gamma, const int32_t* cand,
    const int32_t* len, int32_t* prepared) {
  const int b = blockIdx.x, c = blockIdx.y, nc = 3 * (gamma + 1);
  const size_t slot = (size_t)b * nc + c;
  draft_chain<DT>(table, V, H, noise, P, gamma, cand[slot], (len ? len[b] : 0) + c / 3 + 1,
                  prepared + slot * gamma);
}

// After the verification of a round: the committed state (last token y,
// length) and the next round's drafts, copied from the prepared ones when the
// outcome was predicted (hit[b] set) and drawn afresh otherwise.  A sequence
// the verification marked invalid stays invalid (last token and drafts -1).
template <int DT>
__global__ __launch_bounds__(kChainThreads) void advance_kernel(
    const void* table, int V, int H, const float* noise, int P, int gamma,
    const int32_t* out_tokens, const int32_t* accepted, const int32_t* out_len, const int32_t* hit, const int32_t* cand_idx,
    const int32_t* prepared, int32_t* next_last, int32_t* next_len, int32_t* next_tokens) {
  const int b = blockIdx.x, nc = 3 * (gamma + 1);
  const int k = accepted[b];
  const int len = out_len[b];
  int32_t* dst = next_tokens + (size_t)b * gamma;
  const int y = (k >= 0 && k <= gamma) ? out_tokens[(size_t)b * (gamma + 1) + k] : -1;
  if (threadIdx.x == 0) {
    next_last[b] = y;
    next_len[b] = len;
  }
  const int idx = (hit && prepared && hit[b] != 0) ? cand_idx[b] : -1;
  if (y >= 0 && idx >= 0 && idx < nc) {
    const int32_t* src = prepared + ((size_t)b * nc + idx) * gamma;
    for (int i = threadIdx.x; i < gamma; i += kChainThreads) dst[i] = src[i];
    return;
  }
  draft_chain<DT>(table, V, H, noise, P, gamma, y, len, dst);
}

// Rows [B][gamma+1][V] of a bigram table for one round: row i of sequence b
// follows the token before position i (last[b] for i = 0, tokens[b][i-1]
// after).  A row that follows an invalid token is filled with NaN.  Grid:
// (rows, chunks of kRowChunk elements); 16-byte copies when the rows allow.
template <int DT>
__global__ __launch_bounds__(kRowThreads) void rows_kernel(
    const void* table, int V, int H, int gamma, const int32_t* last, const int32_t* tokens,
    void* out) {
  using E = typename std::conditional<DT == SPEC_BF16, uint16_t, uint32_t>::type;
  constexpr int W = 16 / sizeof(E);
  const int r = blockIdx.x;
  const int b = r / (gamma + 1), i = r % (gamma + 1);
  const int prev = i == 0 ? last[b] : tokens[(size_t)b * gamma + i - 1];
  const int j0 = blockIdx.y * kRowChunk;
  const int j1 = min(V, j0 + kRowChunk);
  E* dst = static_cast<E*>(out) + (size_t)r * V;
  if (prev < 0 || prev >= V) {
    const E nan = DT == SPEC_BF16 ? (E)0x7FC0u : (E)0x7FC00000u;
    for (int j = j0 + threadIdx.x; j < j1; j += kRowThreads) dst[j] = nan;
    return;
  }
  const E* src = static_cast<const E*>(table) + (size_t)((unsigned)prev % (unsigned)H) * V;
  if (V % W == 0 && (((uintptr_t)table | (uintptr_t)out) & 15) == 0) {
    // kRowChunk and V are multiples of W, so j0 and j1 are too
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    uint4* d4 = reinterpret_cast<uint4*>(dst);
    for (int v = j0 / W + threadIdx.x; v < j1 / W; v += kRowThreads) d4[v] = s4[v];
  } else {
    for (int j = j0 + threadIdx.x; j < j1; j += kRowThreads) dst[j] = src[j];
  }
}

bool bigram_args_ok(const void* table, int dtype, int V, int H, const float* noise, int P,
                    int gamma) {
  return table && noise && V >= 1 && V <= kMaxV && H >= 1 && P >= 1 && gamma >= 1 && gamma <= 63 &&
         (dtype == SPEC_F32 || dtype == SPEC_BF16);
}

int launched() { return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH; }

}  // namespace
}  // namespace sv

extern "C" int spec_synth_draft(const void* table, int dtype, int V, int H, const float* noise, int P,
                                int gamma, int n, const int32_t* start_tok,
                                const int32_t* start_pos, int32_t* out_tokens, void* stream) {
  if (!sv::bigram_args_ok(table, dtype, V, H, noise, P, gamma) || n < 0) return SPEC_EINVAL;
  if (n == 0) return SPEC_OK;
  if (!start_tok || !out_tokens) return SPEC_EINVAL;
  (void)hipGetLastError();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(sv::draft_kernel<SPEC_BF16>, dim3(n), dim3(sv::kChainThreads), 0, st,
                       table, V, H, noise, P, gamma, start_tok, start_pos, out_tokens);
  else
    hipLaunchKernelGGL(sv::draft_kernel<SPEC_F32>, dim3(n), dim3(sv::kChainThreads), 0, st,
                       table, V, H, noise, P, gamma, start_tok, start_pos, out_tokens);
  return sv::launched();
}

extern "C" int spec_synth_rows(const void* table, int dtype, int V, int H, int gamma, int B,
                               const int32_t* last, const int32_t* tokens, void* out_rows,
                               void* stream) {
  if (!table || H < 1 || !sv::sizes_in_range(B, gamma, V) ||
      (dtype != SPEC_F32 && dtype != SPEC_BF16))
    return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!last || !tokens || !out_rows) return SPEC_EINVAL;
  (void)hipGetLastError();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)B * (unsigned)(gamma + 1), (V + sv::kRowChunk - 1) / sv::kRowChunk);
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(sv::rows_kernel<SPEC_BF16>, grid, dim3(sv::kRowThreads), 0, st, table, V,
                       H, gamma, last, tokens, out_rows);
  else
    hipLaunchKernelGGL(sv::rows_kernel<SPEC_F32>, grid, dim3(sv::kRowThreads), 0, st, table, V,
                       H, gamma, last, tokens, out_rows);
  return sv::launched();
}

extern "C" int spec_ssd_prespeculate(const void* table, int dtype, int V, int H, const float* noise,
                                     int P, int gamma, int B, const int32_t* cand,
                                     const int32_t* len, int32_t* prepared, void* stream) {
  if (!sv::bigram_args_ok(table, dtype, V, H, noise, P, gamma) || !sv::sizes_in_range(B, gamma, V))
    return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!cand || !prepared) return SPEC_EINVAL;
  (void)hipGetLastError();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid(B, 3 * (gamma + 1));
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(sv::prespec_kernel<SPEC_BF16>, grid, dim3(sv::kChainThreads), 0, st, table,
                       V, H, noise, P, gamma, cand, len, prepared);
  else
    hipLaunchKernelGGL(sv::prespec_kernel<SPEC_F32>, grid, dim3(sv::kChainThreads), 0, st, table,
                       V, H, noise, P, gamma, cand, len, prepared);
  return sv::launched();
}

extern "C" int spec_ssd_advance(const void* table, int dtype, int V, int H, const float* noise, int P,
                                int gamma, int B, const int32_t* out_tokens,
                                const int32_t* accepted, const int32_t* out_len,
                                const int32_t* hit, const int32_t* cand_idx,
                                const int32_t* prepared, int32_t* next_last, int32_t* next_len,
                                int32_t* next_tokens, void* stream) {
  if (!sv::bigram_args_ok(table, dtype, V, H, noise, P, gamma) || !sv::sizes_in_range(B, gamma, V))
    return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!out_tokens || !accepted || !out_len || !next_last || !next_len || !next_tokens ||
      (hit && (!cand_idx || !prepared)))
    return SPEC_EINVAL;
  (void)hipGetLastError();
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(sv::advance_kernel<SPEC_BF16>, dim3(B), dim3(sv::kChainThreads), 0, st,
                       table, V, H, noise, P, gamma, out_tokens, accepted, out_len, hit, cand_idx,
                       prepared, next_last, next_len, next_tokens);
  else
    hipLaunchKernelGGL(sv::advance_kernel<SPEC_F32>, dim3(B), dim3(sv::kChainThreads), 0, st,
                       table, V, H, noise, P, gamma, out_tokens, accepted, out_len, hit, cand_idx,
                       prepared, next_last, next_len, next_tokens);
  return sv::launched();
}
