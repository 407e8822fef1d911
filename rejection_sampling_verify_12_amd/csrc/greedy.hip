// Greedy verification (the temperature -> 0 limit of the rule) on gfx950.
//
// "Speculative Decoding: small model guesses, large model verifies", section
// 3 (accept, stop at the first rejection, emit a correction) and section 5.4
// (the rule follows the sampling temperature); "SSSD: Simply-Scalable
// Speculative Decoding", training-strategy section (speculation in greedy and
// in sampling mode).  At T -> 0 the target's distribution at position i is a
// point mass on its largest logit: draft token x_i is accepted iff it is that
// token (lowest id among equal logits), and the token emitted at the stopping
// position k is the target's argmax there (the correction when k < gamma, the
// bonus from row gamma when k == gamma).  Only target rows are read.
//
// One kernel, two kinds of work-group item in a sequence-major order:
//   stream (sequence b, row r <= gamma, chunk c): the chunk's argmax as a
//     64-bit key (order-preserving logit bits over the complemented index, so
//     the largest key is the largest logit with the lowest id), or a NaN
//     marker, handed over through a device-coherent slot;
//   final (sequence b), LAG steps later: merges the slots of its rows, decides
//     the gamma positions with one wave ballot and writes the outputs.
// Blocks are dispatched in order, so a final item only waits for stream items
// that were dispatched before it and never wait themselves: every poll ends.
#include <atomic>
#include "common.h"
#include "spec_verify.h"
#include "topk.h"

#include <limits.h>

#include <algorithm>
#include <cmath>

#undef SV_FILE
#define SV_FILE 7

namespace sv {
namespace {

// Lag of the final items behind their sequence's stream items, in thousandths
// of a round (as many stream items as the GPU holds at once).
#ifndef SV_GREEDY_LAG
#define SV_GREEDY_LAG 1500
#endif

constexpr unsigned kGreedyPolls = 1u << 22;
constexpr uint64_t kNanKey = 1;   // below every element's key

struct GreedyArgs {
  const void* target;
  const int32_t* tokens;
  const int32_t* in_len;
  int32_t* out_tokens;
  int32_t* out_acc;
  int32_t* out_fr;
  uint64_t* out_mask;
  int32_t* out_len;
  unsigned* err;    // nonzero once a bounded wait timed out
  uint64_t* slot;   // [B][gamma+1][nc]: ~key of the chunk's argmax (~kNanKey: NaN); 0 = empty
  int B, gamma, V, nc, chunk;
  int per_seq;      // stream items per sequence, (gamma+1) * nc
  int lag;          // steps between a sequence's stream items and its final item
#if SV_CHECKS
  unsigned* chk;    // the workspace's second word: site of the first failed check
  int64_t n_slot, n_tokens, n_in_len, n_out_tokens, n_out_acc, n_out_fr, n_out_mask, n_out_len;
#endif
};

// Eight logits of a lane (unit start j0): the lane's running maximum and the
// index of its first occurrence (elements arrive in increasing index order,
// so a strict comparison keeps the lowest id), and a NaN flag.
template <int DT, bool VEC>
__device__ __forceinline__ void argmax8(const Raw8<DT, VEC>& raw, int j0, int64_t end, bool full,
                                        float& mx, int& ix, bool& nan) {
  float v[8];
  unpack<DT, VEC>(raw, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool in = full || j0 + e < end;
    nan = nan || (in && v[e] != v[e]);
    if (in && v[e] > mx) {
      mx = v[e];
      ix = j0 + e;
    }
  }
}

struct GreedyLds {
  uint64_t key[kWaves];
  int nan[kWaves];
  uint64_t row[64];   // merged key per row (gamma + 1 <= 64)
};

template <int DT, bool VEC, int U>
__device__ void greedy_stream(const GreedyArgs& a, int b, int r, int c, GreedyLds& sh) {
  constexpr int kEs = DT == kBF16 ? 2 : 4;
#if SV_CHECKS
  b = (int)SV_IDX(a, b, a.B);
  r = (int)SV_IDX(a, r, a.gamma + 1);
  c = (int)SV_IDX(a, c, a.nc);
#endif
  const int64_t ridx = (int64_t)b * (a.gamma + 1) + r;
  const void* row = static_cast<const char*>(a.target) + ridx * a.V * kEs;
  const int64_t begin = (int64_t)c * a.chunk;
  const int64_t end = min<int64_t>(begin + a.chunk, a.V);
  constexpr int64_t kStep = (int64_t)kThreads * kUnit, kBatch = U * kStep;
  // A lane with at least one unit starts at its first element with -inf, so
  // that an all -inf lane reports its lowest id.
  int64_t j = begin + (int64_t)threadIdx.x * kUnit;
  const bool has = j < end;
  float mx = -INFINITY;
  int ix = (int)j;
  bool nan = false;
  if constexpr (VEC) {
    const int nb = (int)((end - begin) / kBatch);
    const __amdgpu_buffer_rsrc_t rs =
        chunk_rsrc(static_cast<const char*>(row) + begin * kEs, (int)((end - begin) * kEs));
    const int voff = (int)threadIdx.x * kUnit * kEs;
    for (int i = 0; i < nb; ++i) {
      Raw8<DT, VEC> raw[U];
#pragma unroll
      for (int u = 0; u < U; ++u) load_raw_buf<DT>(rs, voff, (int)((i * kBatch + u * kStep) * kEs), raw[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) argmax8<DT, VEC>(raw[u], (int)(j + i * kBatch + u * kStep), end, true, mx, ix, nan);
    }
    j += nb * kBatch;
  }
  for (; j < end; j += kStep) {   // the rest, unit by unit, bounds-checked
    Raw8<DT, VEC> raw;
    load_raw<DT, VEC, true>(row, j, end, raw);
    argmax8<DT, VEC>(raw, (int)j, end, false, mx, ix, nan);
  }
  const uint64_t key = wave_max_u64(has ? make_key(__float_as_uint(mx), ix) : 0ull);
  const bool wn = __ballot(nan) != 0;
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.key[w] = key;
    sh.nan[w] = wn ? 1 : 0;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t k = 0;
    int any = 0;
    for (int i = 0; i < kWaves; ++i) {
      k = sh.key[i] > k ? sh.key[i] : k;
      any |= sh.nan[i];
    }
    st_dev_u64(SV_AT(a, slot, ridx * a.nc + c), ~(any ? kNanKey : k));
  }
}

// A slot's word, or ~kNanKey when the wait gives up: the row then counts as
// holding a NaN, so nothing is taken from it.
__device__ __forceinline__ uint64_t greedy_poll(const GreedyArgs& a, const uint64_t* p) {
  uint64_t w = ld_dev_u64(p);
  unsigned polls = 0;
  while (w == 0ull) {
    ++polls;
    if ((polls & 63u) == 0u &&
        (polls > kGreedyPolls || __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
      __hip_atomic_store(a.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return ~kNanKey;
    }
    __builtin_amdgcn_s_sleep(2);
    w = ld_dev_u64(p);
  }
  return w;
}

__device__ void greedy_final(const GreedyArgs& a, int b, GreedyLds& sh) {
  const int G1 = a.gamma + 1;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // The error word, read early so its latency overlaps the polls.
  const unsigned err = __hip_atomic_load(a.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // Rows by wave, chunks by lane: every slot is polled, consumed and cleared.
  for (int r = wave; r < G1; r += kWaves) {
    uint64_t best = 0;
    bool nan = false;
    uint64_t* p = SV_AT(a, slot, ((int64_t)b * G1 + r) * a.nc);
    for (int c = lane; c < a.nc; c += 64) {
      const uint64_t k = ~greedy_poll(a, p + c);
      st_dev_u64(p + c, 0ull);
      if (k == kNanKey) nan = true;
      else best = k > best ? k : best;
    }
    best = wave_max_u64(best);
    nan = __ballot(nan) != 0;
    if (lane == 0) sh.row[r] = nan ? kNanKey : best;
  }
  __syncthreads();
  if (wave != 0) return;
  // Wave 0 decides: lane i < gamma tests position i.
  const bool pos = lane < a.gamma;
  const int x = pos ? *SV_AT(a, tokens, ((int64_t)b * a.gamma + lane)) : 0;
  const bool bad_x = pos && (x < 0 || x >= a.V);
  const uint64_t rk = pos ? sh.row[lane] : 0ull;
  const bool nan_i = pos && rk == kNanKey;
  const uint64_t mask = __ballot(pos && !bad_x && !nan_i && key_index(rk) == x);
  // After a bounded wait has given up anywhere in the call (the error word),
  // the sequence is reported invalid.
  bool bad = __ballot(bad_x || nan_i) != 0 || err != 0u;
  const int k = (int)SV_IDX(a, __builtin_ctzll(~mask), G1);   // <= gamma: bit gamma of mask is clear
  const uint64_t ky = sh.row[k];
  if (k == a.gamma && ky == kNanKey) bad = true;
  const int y = key_index(ky);
  if (lane < G1) {
    const int t = bad ? -1 : (lane < k ? x : (lane == k ? y : -1));
    *SV_AT(a, out_tokens, ((int64_t)b * G1 + lane)) = t;
  }
  if (lane == 0) {
    const int in = a.in_len ? *SV_AT(a, in_len, b) : 0;
    *SV_AT(a, out_acc, b) = bad ? -1 : k;
    if (a.out_fr) *SV_AT(a, out_fr, b) = bad ? -1 : (k < a.gamma ? k : -1);
    if (a.out_mask) *SV_AT(a, out_mask, b) = bad ? 0ull : mask;
    if (a.out_len) *SV_AT(a, out_len, b) = bad ? in : in + k + 1;
  }
}

// Item j of the order: step t holds the stream items of sequence t and the
// final item of sequence t - lag.
__device__ __forceinline__ void greedy_decode(const GreedyArgs& a, int64_t j, bool& fin, int& b, int& sub) {
  const int64_t S = a.per_seq;
  auto off = [&](int t) -> int64_t {
    const int64_t ns = std::min<int64_t>(std::max(t, 0), a.B);
    const int64_t nf = std::min<int64_t>(std::max(t - a.lag, 0), a.B);
    return ns * S + nf;
  };
  int lo = 0, hi = a.B + a.lag;   // off(lo) <= j < off(hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off(mid) <= j) lo = mid;
    else hi = mid;
  }
  int64_t w = j - off(lo);
  if (lo < a.B) {
    if (w < S) {
      fin = false;
      b = lo;
      sub = (int)w;
      return;
    }
    w -= S;
  }
  fin = true;
  b = lo - a.lag;
  sub = 0;
}

template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void greedy_kernel(GreedyArgs) {
  const GreedyArgs& a = kernel_arg0<GreedyArgs>();
  __shared__ GreedyLds sh;
  __shared__ int item[3];
  if (threadIdx.x < 64) {
    bool fin;
    int b, sub;
    greedy_decode(a, blockIdx.x, fin, b, sub);
    if (threadIdx.x == 0) {
      item[0] = fin ? 1 : 0;
      item[1] = b;
      item[2] = sub;
    }
  }
  __syncthreads();
  const int fin = uni(item[0]), b = uni(item[1]), sub = uni(item[2]);
#if SV_CHECKS
  if (threadIdx.x == 0) {   // the decoded item: a sequence, and a part of it
    SV_IDX(a, b, a.B);
    SV_IDX(a, sub, fin ? 1 : a.per_seq);
  }
#endif
  if (fin) {
    greedy_final(a, b, sh);
  } else {
    const int r = sub / a.nc, c = sub - r * a.nc;
    greedy_stream<DT, VEC, 4>(a, b, r, c, sh);
  }
}

size_t greedy_bytes(int B, int gamma, int V) {
  if (B == 0) return 0;
  const size_t nc = (size_t)((V + kChunk - 1) / kChunk);
  return 256 + (((size_t)B * (gamma + 1) * nc * sizeof(uint64_t) + 255) & ~(size_t)255);
}

// Work-groups the device holds at once, cached per device.  The entries are
// atomics: concurrent callers may fill one at the same time, with the same
// value.
template <int DT, bool VEC>
hipError_t greedy_slots(int& slots) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::atomic<int>* c = dev >= 0 && dev < 64 ? &cache[dev] : nullptr;
  const int cached = c ? c->load(std::memory_order_relaxed) : 0;
  if (cached > 0) {
    slots = cached;
    return hipSuccess;
  }
  int ncu = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(greedy_kernel<DT, VEC>), kThreads, 0);
  if (e != hipSuccess) return e;
  slots = std::max(1, ncu * per_cu);
  if (c) c->store(slots, std::memory_order_relaxed);
  return hipSuccess;
}

template <int DT, bool VEC>
hipError_t greedy_launch(GreedyArgs a, hipStream_t st) {
  int slots = 0;
  hipError_t e = greedy_slots<DT, VEC>(slots);
  if (e != hipSuccess) return e;
  a.lag = std::max(1, (int)std::lround((double)slots / a.per_seq * SV_GREEDY_LAG / 1000.0));
  const int64_t items = (int64_t)a.B * (a.per_seq + 1);
  hipLaunchKernelGGL((greedy_kernel<DT, VEC>), dim3((unsigned)items), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace sv

extern "C" int spec_verify_greedy(const void* target_logits, int dtype, const int32_t* draft_tokens,
                                  int B, int gamma, int V, const int32_t* in_len, int32_t* out_tokens,
                                  int32_t* out_accepted, int32_t* out_first_reject,
                                  uint64_t* out_accept_mask, int32_t* out_len, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  using namespace sv;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (!sizes_in_range(B, gamma, V)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!target_logits || !draft_tokens || !out_tokens || !out_accepted) return SPEC_EINVAL;
  const int nc = (V + kChunk - 1) / kChunk;
  const int64_t per_seq = (int64_t)(gamma + 1) * nc;
  const int64_t items = (int64_t)B * (per_seq + 1);
  if (items * kThreads > (int64_t)UINT_MAX || per_seq > INT_MAX / 2) return SPEC_EINVAL;
  if (!workspace || workspace_bytes < greedy_bytes(B, gamma, V)) return SPEC_EWORKSPACE;
  GreedyArgs a;
  a.target = target_logits;
  a.tokens = draft_tokens;
  a.in_len = in_len;
  a.out_tokens = out_tokens;
  a.out_acc = out_accepted;
  a.out_fr = out_first_reject;
  a.out_mask = out_accept_mask;
  a.out_len = out_len;
  char* w = static_cast<char*>(workspace);
  a.err = reinterpret_cast<unsigned*>(w);
  a.slot = reinterpret_cast<uint64_t*>(w + 256);
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.nc = nc;
  a.chunk = kChunk;
  a.per_seq = (int)per_seq;
  a.lag = 1;
#if SV_CHECKS
  a.chk = a.err + 1;
  a.n_slot = (int64_t)B * (gamma + 1) * nc;
  a.n_tokens = (int64_t)B * gamma;
  a.n_in_len = in_len ? B : 0;
  a.n_out_tokens = (int64_t)B * (gamma + 1);
  a.n_out_acc = B;
  a.n_out_fr = out_first_reject ? B : 0;
  a.n_out_mask = out_accept_mask ? B : 0;
  a.n_out_len = out_len ? B : 0;
#endif
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool vec = (V % 8 == 0) && ((uintptr_t)target_logits % 16 == 0);
  hipError_t e;
  if (dtype == SPEC_BF16) e = vec ? greedy_launch<kBF16, true>(a, st) : greedy_launch<kBF16, false>(a, st);
  else e = vec ? greedy_launch<kF32, true>(a, st) : greedy_launch<kF32, false>(a, st);
  return e == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

extern "C" size_t spec_greedy_workspace_bytes(int B, int gamma, int V, int dtype) {
  if ((dtype != SPEC_F32 && dtype != SPEC_BF16) || !sv::sizes_in_range(B, gamma, V))
    return 0;
  return sv::greedy_bytes(B, gamma, V);
}
