// Device helpers shared by the verification and outcome-prediction kernels.
// gfx950 (CDNA4): 64-lane wavefronts, 256-thread work-groups (4 waves).
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace sv {

constexpr int kThreads = 256;               // every kernel runs 256-thread work-groups
constexpr int kWaves = kThreads / 64;
constexpr int kUnit = 8;                    // logits per thread per load unit (16 B of bf16)
constexpr int kTile = kThreads * kUnit;     // 2048 logits: granularity of the sampling scan
#ifndef SV_CHUNK
#define SV_CHUNK 32768
#endif
constexpr int kChunk = SV_CHUNK;            // logits of one row per statistics work-group (target)
constexpr float kNegSentinel = -1.0e30f;    // "no finite logit seen yet"

enum : int { kF32 = 0, kBF16 = 1 };

// Sizes every entry point accepts: B >= 0, 1 <= gamma <= 63, 1 <= V <= 2^30,
// and B * (2 gamma + 1) * ceil(V / 2048) <= 2^29 (about 2^40 logits per
// tensor, terabytes beyond one GPU's memory).  Within these limits every row,
// tile, chunk and item count of a call, and every schedule step, fits a
// 32-bit int.
constexpr int kMaxV = 1 << 30;
inline bool sizes_in_range(int B, int gamma, int V) {
  if (B < 0 || gamma < 1 || gamma > 63 || V < 1 || V > kMaxV) return false;
  const int64_t rows = (int64_t)B * (2 * gamma + 1);
  return rows * (((int64_t)V + kTile - 1) / kTile) <= ((int64_t)1 << 29);
}

// ---------------------------------------------------------------------------
// Checks build (SV_CHECKS=1, a separate library).  Every index a kernel forms
// into the workspace, an input or an output array, and every row, chunk and
// tile an item selects, is tested against its array's size before use.  A
// failed test never traps: it records its site (the source file's number,
// below, times 2^16 plus the line) in the call's check word - the first
// failure wins - and the index is clamped into the array, so the access
// stays in bounds and the call runs to its end.  The default build compiles
// the tests out.  Source file numbers: 1 verify_args.h, 2 verify_stream.h,
// 3 verify_decide.h, 4 verify_sample.h, 5 verify_topp.h, 6 verify_kernels.h,
// 7 greedy.hip.  The check word is the workspace's second 32-bit word (the
// first is the error word of the bounded waits); like the error word it stays
// set until the caller clears it.  The stand-alone outcome prediction has no
// check word and no checks.
#ifndef SV_CHECKS
#define SV_CHECKS 0
#endif
#if SV_CHECKS
__device__ __noinline__ int64_t check_failed(unsigned* chk, int64_t i, int64_t n, unsigned site) {
  atomicCAS(chk, 0u, site);
  return i < 0 || n <= 0 ? 0 : n - 1;
}
__device__ __forceinline__ int64_t check_index(unsigned* chk, int64_t i, int64_t n, unsigned site) {
  return (i >= 0 && i < n) ? i : check_failed(chk, i, n, site);
}
#define SV_SITE ((unsigned)SV_FILE << 16 | (unsigned)__LINE__)
// Index i of array n elements long (the index, clamped on failure), and
// element i of array field f of the arguments a, whose length is a.n_f.
#define SV_IDX(a, i, n) ::sv::check_index((a).chk, (int64_t)(i), (int64_t)(n), SV_SITE)
#define SV_AT(a, f, i) ((a).f + SV_IDX(a, i, (a).n_##f))
#else
// The default build leaves every index expression as it was written: i is
// not parenthesised, so a.f + x + y keeps its association (pass a single
// term, a sum or a product; an index written as one unit is parenthesised at
// its call).
#define SV_IDX(a, i, n) (i)
#define SV_AT(a, f, i) ((a).f + i)
#endif

// A kernel's first argument, read where the argument segment holds it
// (explicit arguments start the segment): each field is loaded where it is
// used.  Taken by value, every field a kernel uses is loaded at its entry
// into scalar registers, which then spill to vector lanes on every
// work-group.
template <class T>
__device__ __forceinline__ const T& kernel_arg0() {
  return *(const T*)__builtin_amdgcn_kernarg_segment_ptr();
}

// ---------------------------------------------------------------------------
// Logit loads.  A row is `const void*`; element j is float32 or bfloat16.

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DT>
__device__ __forceinline__ float load_one(const void* row, int64_t j) {
  if constexpr (DT == kBF16) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(row)[j]) << 16);
  } else {
    return static_cast<const float*>(row)[j];
  }
}

// Eight consecutive logits starting at j0.  VEC: j0 + 8 <= n and 16-byte
// aligned rows (one or two 16-byte loads).  Otherwise per-element loads with
// positions >= n read as -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load8(const void* row, int64_t j0, int64_t n, float (&v)[8]) {
  if constexpr (VEC) {
    if constexpr (DT == kBF16) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + j0);
      v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
      v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
      v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
      v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(row) + j0);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (j0 + e < n) ? load_one<DT>(row, j0 + e) : -INFINITY;
  }
}

// Eight logits as loaded: the raw 16-byte word for aligned bf16 rows (unpacked
// when used, so a batch of loads in flight costs 4 VGPRs per eight logits),
// floats otherwise.
template <int DT, bool VEC>
struct Raw8 {
  float v[8];
};
template <>
struct Raw8<kBF16, true> {
  uint4 w;
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// NT: a nontemporal load (data read once: streamed through the caches
// without being kept; reads noticeably faster from HBM on gfx950).
template <int DT, bool VEC, bool NT = false>
__device__ __forceinline__ void load_raw(const void* row, int64_t j0, int64_t n, Raw8<DT, VEC>& r) {
  if constexpr (DT == kBF16 && VEC) {
    if (j0 < n) {
      const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(row) + j0);
      const u32x4 t = NT ? __builtin_nontemporal_load(p) : *p;
      r.w = make_uint4(t.x, t.y, t.z, t.w);
    } else {
      r.w = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);   // -inf
    }
  } else if constexpr (DT == kF32 && VEC && NT) {
    if (j0 < n) {
      const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(row) + j0);
      const f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
      r.v[0] = a.x; r.v[1] = a.y; r.v[2] = a.z; r.v[3] = a.w;
      r.v[4] = b.x; r.v[5] = b.y; r.v[6] = b.z; r.v[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r.v[e] = -INFINITY;
    }
  } else {
    if (j0 < n) {
      load8<DT, VEC>(row, j0, n, r.v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r.v[e] = -INFINITY;
    }
  }
}

// Eight logits of an aligned row through a buffer resource: the lane's byte
// offset `voff` stays in a vector register and the batch offset `soff` is
// scalar, so stepping through a chunk costs no vector instructions.
// Nontemporal (read once).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
template <int DT>
__device__ __forceinline__ void load_raw_buf(__amdgpu_buffer_rsrc_t rs, int voff, int soff,
                                             Raw8<DT, true>& r) {
  constexpr int kNT = 2;   // cache policy: nontemporal
  if constexpr (DT == kBF16) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kNT);
    r.w = make_uint4(t.x, t.y, t.z, t.w);
  } else {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kNT);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff, kNT);
    r.v[0] = __uint_as_float(a.x); r.v[1] = __uint_as_float(a.y);
    r.v[2] = __uint_as_float(a.z); r.v[3] = __uint_as_float(a.w);
    r.v[4] = __uint_as_float(b.x); r.v[5] = __uint_as_float(b.y);
    r.v[6] = __uint_as_float(b.z); r.v[7] = __uint_as_float(b.w);
  }
}

template <int DT, bool VEC>
__device__ __forceinline__ void unpack(const Raw8<DT, VEC>& r, float (&v)[8]) {
  if constexpr (DT == kBF16 && VEC) {
    v[0] = bf16_lo(r.w.x); v[1] = bf16_hi(r.w.x);
    v[2] = bf16_lo(r.w.y); v[3] = bf16_hi(r.w.y);
    v[4] = bf16_lo(r.w.z); v[5] = bf16_hi(r.w.z);
    v[6] = bf16_lo(r.w.w); v[7] = bf16_hi(r.w.w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = r.v[e];
  }
}

// A value equal in every lane, moved to a scalar register (frees vector
// registers on long paths).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
__device__ __forceinline__ uint64_t uni(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double uni(double x) {
  return __longlong_as_double((long long)uni((uint64_t)__double_as_longlong(x)));
}

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Cross-work-group hand-off without cache-wide maintenance.  A producer
// writes its payload with device-coherent (agent-scope) stores, waits until
// they have completed, then bumps an arrival counter with a relaxed atomic;
// the consumer reads payloads with device-coherent loads.  (An agent-scope
// fence would write back and invalidate the whole L2 of the XCD instead.)

__device__ __forceinline__ void st_dev(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p),
                     (unsigned long long)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_dev(const double* p) {
  return __longlong_as_double((long long)__hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_dev_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), (unsigned long long)v,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev_u64(const uint64_t* p) {
  return (uint64_t)__hip_atomic_load(reinterpret_cast<const unsigned long long*>(p),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait for every outstanding memory operation of this wave (s_waitcnt 0).
__device__ __forceinline__ void wait_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------
// Cross-lane steps through DPP: a VALU move whose source lane is permuted
// within a row of 16 lanes, shifted, or broadcast from one row to the next -
// a few cycles, against the LDS round trip of a lane permute (a 64-bit value
// takes two moves either way).  Controls in the GFX9 encoding.
#ifndef SV_DPP
#define SV_DPP 1
#endif
enum : int {
  kDppQuad1032 = 0xB1,       // quad_perm [1,0,3,2]: lane ^ 1
  kDppQuad2301 = 0x4E,       // quad_perm [2,3,0,1]: lane ^ 2
  kDppRowShr = 0x110,        // + n: lane - n within the row
  kDppWaveShr1 = 0x138,      // lane - 1 across the wave
  kDppRowMirror = 0x140,     // lane 15 - i of the row
  kDppRowHalfMirror = 0x141, // lane 7 - i of the half-row
  kDppRowBcast15 = 0x142,    // lane 15 of each row into the next row
  kDppRowBcast31 = 0x143,    // lane 31 into rows 2 and 3
};
// Lanes the controls, the row mask or the bank mask leave out take `old`
// (or 0 with BC, for a source outside the row or wave).
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF, bool BC = false>
__device__ __forceinline__ int dpp(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, BANKS, BC);
}
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF, bool BC = false>
__device__ __forceinline__ float dpp(float v, float old) {
  return __int_as_float(dpp<CTRL, ROWS, BANKS, BC>(__float_as_int(v), __float_as_int(old)));
}
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF, bool BC = false>
__device__ __forceinline__ double dpp(double v, double old) {
  const uint64_t x = (uint64_t)__double_as_longlong(v), o = (uint64_t)__double_as_longlong(old);
  const uint32_t lo = (uint32_t)dpp<CTRL, ROWS, BANKS, BC>((int)(uint32_t)x, (int)(uint32_t)o);
  const uint32_t hi = (uint32_t)dpp<CTRL, ROWS, BANKS, BC>((int)(uint32_t)(x >> 32), (int)(uint32_t)(o >> 32));
  return __longlong_as_double((long long)((uint64_t)hi << 32 | lo));
}
// op over each row of 16 lanes, in every lane of the row (the row's lanes
// all active).
template <class T, class Op>
__device__ __forceinline__ T row16_reduce(T v, Op op) {
  v = op(v, dpp<kDppQuad1032>(v, v));
  v = op(v, dpp<kDppQuad2301>(v, v));
  v = op(v, dpp<kDppRowHalfMirror>(v, v));
  return op(v, dpp<kDppRowMirror>(v, v));
}
// Pair each lane with its lane in the other row of its 32-lane half
// (SWAP 16) or in the other half (SWAP 32): both lanes of a pair get the
// pair's two values, the lower row's (half's) first, so they combine the same
// values in the same order.
template <int SWAP>
__device__ __forceinline__ int2 swap_pair(int v) {
  const auto r = SWAP == 16 ? __builtin_amdgcn_permlane16_swap(v, v, false, false)
                            : __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return make_int2((int)r[0], (int)r[1]);
}
template <int SWAP, class Op>
__device__ __forceinline__ float swap_combine(float v, Op op) {
  const int2 p = swap_pair<SWAP>(__float_as_int(v));
  return op(__int_as_float(p.x), __int_as_float(p.y));
}
template <int SWAP, class Op>
__device__ __forceinline__ int swap_combine(int v, Op op) {
  const int2 p = swap_pair<SWAP>(v);
  return op(p.x, p.y);
}
template <int SWAP, class Op>
__device__ __forceinline__ double swap_combine(double v, Op op) {
  const uint64_t x = (uint64_t)__double_as_longlong(v);
  const int2 lo = swap_pair<SWAP>((int)(uint32_t)x), hi = swap_pair<SWAP>((int)(uint32_t)(x >> 32));
  const double a = __longlong_as_double((long long)((uint64_t)(uint32_t)hi.x << 32 | (uint32_t)lo.x));
  const double b = __longlong_as_double((long long)((uint64_t)(uint32_t)hi.y << 32 | (uint32_t)lo.y));
  return op(a, b);
}
// op over the wave (every lane active), the same value in every lane, kept in
// vector registers: rows of 16 by DPP, then the row pairs and the halves by
// the gfx950 lane swaps.
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = row16_reduce(v, op);
  v = swap_combine<16>(v, op);
  return swap_combine<32>(v, op);
}

// Wave reductions through LDS lane permutes.
__device__ __forceinline__ double wave_sum_lds(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max_lds(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ---------------------------------------------------------------------------
// Work-group reductions and scans (256 threads, 4 waves).  `lds` must hold
// kWaves entries of the reduced type; each call ends with a barrier so the
// scratch can be reused.

__device__ __forceinline__ double wave_sum(double v) {
#if SV_DPP
  return wave_reduce(v, [](double x, double y) { return x + y; });
#else
  return wave_sum_lds(v);
#endif
}

__device__ __forceinline__ float wave_max(float v) {
#if SV_DPP
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
#else
  return wave_max_lds(v);
#endif
}

__device__ __forceinline__ int wave_min_int(int v) {
#if SV_DPP
  return wave_reduce(v, [](int x, int y) { return min(x, y); });
#else
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
#endif
}

// Inclusive prefix sum over the wave (every lane active).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
#if SV_DPP
  double s = v + dpp<kDppRowShr + 1, 0xF, 0xF, true>(v, 0.0);
  s += dpp<kDppRowShr + 2, 0xF, 0xF, true>(v, 0.0);
  s += dpp<kDppRowShr + 3, 0xF, 0xF, true>(v, 0.0);          // rows: sums of 4
  s += dpp<kDppRowShr + 4, 0xF, 0xE>(s, 0.0);                // lanes 4..15 of a row
  s += dpp<kDppRowShr + 8, 0xF, 0xC>(s, 0.0);                // lanes 8..15
  s += dpp<kDppRowBcast15, 0xA>(s, 0.0);                     // rows 1, 3
  s += dpp<kDppRowBcast31, 0xC>(s, 0.0);                     // rows 2, 3
  return s;
#else
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o, 64);
    if (l >= o) v += t;
  }
  return v;
#endif
}

__device__ __forceinline__ double block_sum(double v, double* lds) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) lds[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += lds[i];
  __syncthreads();
  return t;
}

// N sums at once (one barrier pair); lds holds kWaves * N doubles.
template <int N>
__device__ __forceinline__ void block_sum_n(double (&v)[N], double* lds) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) lds[w * N + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double t = 0.0;
#pragma unroll
    for (int j = 0; j < kWaves; ++j) t += lds[j * N + i];
    v[i] = t;
  }
  __syncthreads();
}

// N maxima at once (one barrier pair); lds holds kWaves * N floats.
template <int N>
__device__ __forceinline__ void block_max_n(float (&v)[N], float* lds) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_max(v[i]);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) lds[w * N + i] = v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float t = lds[i];
#pragma unroll
    for (int j = 1; j < kWaves; ++j) t = fmaxf(t, lds[j * N + i]);
    v[i] = t;
  }
  __syncthreads();
}

__device__ __forceinline__ float block_max(float v, float* lds) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) lds[w] = v;
  __syncthreads();
  float t = lds[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) t = fmaxf(t, lds[i]);
  __syncthreads();
  return t;
}

__device__ __forceinline__ int block_min_int(int v, int* lds) {
  v = wave_min_int(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) lds[w] = v;
  __syncthreads();
  int t = lds[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) t = min(t, lds[i]);
  __syncthreads();
  return t;
}

// Exclusive prefix sum over the work-group in thread order; returns this
// thread's offset and writes the total.
__device__ __forceinline__ double block_exclusive_scan(double v, double* lds, double& total) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const double incl = wave_inclusive_scan(v);
  __syncthreads();
  if (l == 63) lds[w] = incl;
  __syncthreads();
  double before = 0.0, all = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) before += lds[i];
    all += lds[i];
  }
  __syncthreads();
  total = all;
#if SV_DPP
  const double excl = dpp<kDppWaveShr1, 0xF, 0xF, true>(incl, 0.0);
#else
  const double excl = __shfl_up(incl, 1, 64);
#endif
  return before + (l == 0 ? 0.0 : excl);
}

}  // namespace sv
