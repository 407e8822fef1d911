// Top-p: each row's nucleus by radix selection (float32) or by counting (bfloat16).
#pragma once
#include "verify_kernels.h"

#undef SV_FILE
#define SV_FILE 5

namespace sv {

// ---------------------------------------------------------------------------
// Top-p: the nucleus threshold of every row by a radix selection over the
// logits' order-preserving keys (16 bits for bfloat16, 32 for float32; 8 bits
// a pass), each key weighted by its probability mass, from the highest key
// down, until the mass reaches top_p.

// The order-preserving key of a logit (+0.0 and -0.0 share one), in kb bits.
template <int DT>
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  const uint32_t k = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return DT == kBF16 ? k >> 16 : k;
}
template <int DT>
__device__ __forceinline__ float key_logit(uint32_t k) {
  if constexpr (DT == kBF16) {
    const uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
    return __uint_as_float(b << 16);
  } else {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
  }
}

// One wave per row: the row's offset and normaliser from its pieces (left in
// place for the decision), and the selection's start.
__global__ __launch_bounds__(64) void topp_init_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const uint64_t* p = SV_AT(a, part, row * a.nc);
  double M = -INFINITY;
  for (int c = lane; c < a.nc; c += 64) M = fmax(M, slot_value(ld_dev_u64(p + c)));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmax(M, __shfl_xor(M, o, 64));
  M = ceil(M);
  double z = 0.0;
  for (int c = lane; c < a.nc; c += 64) {
    const double v = slot_value(ld_dev_u64(p + c));
    if (v != -INFINITY) z += exp2(v - M);
  }
  z = wave_sum(z);
  if (lane == 0) {
    TopPRow t;
    t.M = M;
    t.Z = z;
    t.rem = (double)a.top_p * z;
    t.above = 0.0;
    t.P = 1.0;
    t.prefix = 0u;
    t.L = -INFINITY;
    *SV_AT(a, topp, row) = t;
  }
}

// (row, chunk) items: the masses of the chunk's logits whose key matches the
// selected prefix, by the pass's digit, into the row's histogram.  Each wave
// has its own LDS histogram (fewer colliding atomics); a lane sums runs of
// one digit before adding.  Loads: four units in flight per lane.
template <int DT, bool VEC>
__global__ __launch_bounds__(kThreads) void topp_hist_kernel(VerifyArgs, int pass) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ double h[kWaves][kDigits];
  const int R = 2 * a.gamma + 1;
  const int64_t id = blockIdx.x;
  const int64_t row = id / a.nc;
  const int c = (int)(id - row * a.nc);
  const int b = (int)(row / R), r = (int)(row - (int64_t)b * R);
  const TCoef tc = temp_coef(a, b);
  const float Mf = (float)uni(SV_AT(a, topp, row)->M);
  const uint32_t prefix = (uint32_t)uni((int)SV_AT(a, topp, row)->prefix);
  constexpr int KB = DT == kBF16 ? 16 : 32;
  const int shift = KB - 8 * (pass + 1);
  const int wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kWaves * kDigits; i += kThreads) (&h[0][0])[i] = 0.0;
  __syncthreads();
  const void* rp = row_ptr<DT>(a, b, r);
  const int64_t begin = (int64_t)c * a.chunk;
  const int64_t end = min<int64_t>(begin + a.chunk, a.V);
  int cur = -1;
  double acc = 0.0;
  auto take = [&](const Raw8<DT, VEC>& raw, int64_t j) {
    float v[8];
    unpack<DT, VEC>(raw, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (j + e >= end) continue;
      const uint32_t key = logit_key<DT>(v[e]);
      if (pass > 0 && (key >> (shift + 8)) != prefix) continue;
      const int d = (int)((key >> shift) & 0xFFu);
      const double m = (double)exp2_fast(fmaf(v[e], tc.c_lo, fmaf(v[e], tc.c_hi, -Mf)));
      if (d != cur) {
        if (cur >= 0) atomicAdd(&h[wave][cur], acc);
        cur = d;
        acc = 0.0;
      }
      acc += m;
    }
  };
  constexpr int U = 4;
  int64_t j = begin + (int64_t)threadIdx.x * kUnit;
  for (; j + (U - 1) * (int64_t)kTile < end; j += U * (int64_t)kTile) {
    Raw8<DT, VEC> raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load_raw<DT, VEC, true>(rp, j + u * (int64_t)kTile, end, raw[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) take(raw[u], j + u * (int64_t)kTile);
  }
  for (; j < end; j += kTile) {
    Raw8<DT, VEC> raw;
    load_raw<DT, VEC, true>(rp, j, end, raw);
    take(raw, j);
  }
  if (cur >= 0) atomicAdd(&h[wave][cur], acc);
  __syncthreads();
  double* g = SV_AT(a, hist, row * kDigits);
  for (int i = threadIdx.x; i < kDigits; i += kThreads) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) t += h[w][i];
    if (t != 0.0) atomicAdd(g + i, t);
  }
}

// One wave per row: the digit at which the mass from the top reaches the
// remaining target; clears the histogram.  Lane l holds digits 4l..4l+3 and
// a suffix sum over the lanes gives the mass above each lane's digits.  If
// rounding left the target above the row's total, every digit is kept (the
// lowest digit with mass is selected).  After the last pass, the threshold
// logit and the nucleus mass.
template <int DT>
__global__ __launch_bounds__(64) void topp_select_kernel(VerifyArgs, int pass, int npass) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  TopPRow t = *SV_AT(a, topp, row);
  double* g = SV_AT(a, hist, row * kDigits);
  double m[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) m[q] = g[4 * lane + q];
#pragma unroll
  for (int q = 0; q < 4; ++q) g[4 * lane + q] = 0.0;
  const double mine = (m[0] + m[1]) + (m[2] + m[3]);
  double incl = mine;   // inclusive suffix sum over the lanes (higher digits)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double x = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += x;
  }
  const double above_lane = incl - mine;
  // In this lane, from its highest digit down: the first that reaches the target.
  int sel = -1;
  double run = above_lane, hsel = 0.0, before = 0.0;
#pragma unroll
  for (int q = 3; q >= 0; --q) {
    if (sel < 0 && m[q] > 0.0 && run + m[q] >= t.rem) {
      sel = 4 * lane + q;
      hsel = m[q];
      before = run;
    }
    if (sel < 0) run += m[q];
  }
  // The lowest digit with mass in this lane, for the keep-everything case.
  int low = -1;
  double low_h = 0.0, low_before = 0.0;
  {
    double r2 = above_lane;
#pragma unroll
    for (int q = 3; q >= 0; --q) {
      if (m[q] > 0.0) {
        low = 4 * lane + q;
        low_h = m[q];
        low_before = r2;
      }
      r2 += m[q];
    }
  }
  const uint64_t has = __ballot(sel >= 0);
  const uint64_t haslow = __ballot(low >= 0);
  int src, s_sel;
  double s_h, s_before;
  if (has) {   // the highest digit (lane) that reaches the target
    src = 63 - __builtin_clzll(has);
    s_sel = __shfl(sel, src, 64);
    s_h = __shfl(hsel, src, 64);
    s_before = __shfl(before, src, 64);
  } else {     // keep everything down to the lowest digit with mass
    src = haslow ? __builtin_ctzll(haslow) : 0;
    s_sel = haslow ? __shfl(low, src, 64) : 0;
    s_h = haslow ? __shfl(low_h, src, 64) : 0.0;
    s_before = haslow ? __shfl(low_before, src, 64) : 0.0;
  }
  if (lane == 0) {
    t.above += s_before;
    t.rem -= s_before;
    t.prefix = (t.prefix << 8) | (uint32_t)s_sel;
    if (pass == npass - 1) {
      t.L = key_logit<DT>(t.prefix);
      t.P = (t.above + s_h) / t.Z;
    }
    *SV_AT(a, topp, row) = t;
  }
}


// Top-p of bfloat16 rows by counting.  A bfloat16 row holds at most 65536
// distinct values and every logit of one value carries the same mass, so the
// row's masses in value order follow exactly from how often each value
// occurs.  For each row a 1024-thread work-group (all 128 KB of counters
// fill its CU's LDS):
//   * counts the row's values in LDS, two 16-bit counters per 32-bit word,
//     so that neighbouring values, which a row's logits crowd, fall in
//     different words: topp_count_kernel by the raw bits x (word x & 0x7FFF,
//     the low half for a non-negative value, the high half for a negative
//     one; the crowded values in per-lane copies, the band, below), and
//     topp_redo_kernel by the 16-bit order-preserving keys (word w counts
//     key w, a negative value, in its low half and key w + 32768, a
//     non-negative one, in its high half).  A counter wraps only where one
//     value occurs 65536 times or more; the counters then sum to less than
//     V, and the row is counted again (topp_redo_kernel) with returning
//     atomics that record every wrap, so only such rows are read a second
//     time;
//   * from the counts, from the top value down: the largest finite value (the
//     row offset), the row normaliser in fp64, and the nucleus threshold (the
//     first value at whose end the running mass reaches top_p times the
//     normaliser; each value is one run of equal logits);
//   * writes the row's normaliser piece (the whole row in piece 0, -inf in
//     the others) and its maximum where the stream items would, so a cut
//     bfloat16 row needs no stream items.
constexpr int kCountThreads = 1024;
constexpr int kCountWaves = kCountThreads / 64;
constexpr int kCountWords = 32768;                                     // 128 KB of counters
constexpr int kWordsPerThread = kCountWords / kCountThreads;           // 32
// Wraps in a row of V logits: at most V / 65536 of low counters, plus
// (V + those) / 65536 of high counters (each low wrap carries one into the
// high counter of its word): at most 257 up to this row length, within the
// kCountEvents the checked pass records.  Longer bfloat16 rows take the
// radix selection.
constexpr int64_t kCountMaxV = (int64_t)1 << 24;
constexpr int kCountEvents = 288;
constexpr uint32_t kKeyNegInf = 0x007Fu, kKeyNegZero = 0x7FFFu, kKeyPosZero = 0x8000u,
                   kKeyPosInf = 0xFF80u;

// The counted row's raw words with a count, compacted in ascending order
// (word, low count | high count << 16) for the wave that finishes the row
// while the next one is counted; a row with more is left to
// topp_redo_kernel.
constexpr int kListCap = 1792;
// The band: the 64 raw values from a row's origin up (set just below the
// median of a sample of the row, where its logits crowd) are counted in
// per-lane copies, so the lanes of one add reach 64 different words and
// banks (an LDS atomic add takes two clocks for each lane on its most loaded
// bank, lanes on one word included).  Word 64 i + l holds value origin + i
// for lane l of every counting wave, in the half its counter takes; a copy
// takes at most (V / 960 + 9) * 15 < 65536 counts for rows up to kBandMaxV.
// After the row the copies are summed into the counters.
#ifndef SV_COUNT_PIPE
#define SV_COUNT_PIPE 2
#endif
constexpr int kBandKeys = 64;
constexpr int kBandWords = kBandKeys * 64;
constexpr int64_t kBandMaxV = (int64_t)1 << 21;
constexpr uint32_t kBandOff = 0x10000u;   // an origin no key reaches: no band
constexpr unsigned kRedoWrapped = 0x80000000u;   // a redo entry's flag: the row's counters wrapped
constexpr int kCountingWaves = kCountWaves - 1;
constexpr int kCountingThreads = 64 * kCountingWaves;

struct CountLds {
  uint32_t cnt[kCountWords + kBandWords];   // the counters, then the band's copies
  uint2 list[kListCap];
  uint32_t ev[kCountEvents];   // keys whose counter wrapped (checked pass)
  uint32_t nev;
  uint32_t sum[kCountWaves], nzw[kCountWaves];
  int kmax[kCountWaves], flags[kCountWaves];
  double tot[2][kCountWaves];
  int sel;
  double P;
  uint32_t org[2];   // band origins: row n of the work-group counts with org[n & 1]
};

// The keys of the two bfloat16 logits in w (its halves), in the halves of
// the result: a negative value's bits inverted, a non-negative value's sign
// bit set.  -0 takes key 0x7FFF, next below +0's 0x8000; both are the value
// zero and are merged when the counts are read.
__device__ __forceinline__ uint32_t bf16_key_pair(uint32_t w) {
  const uint32_t s = w & 0x80008000u;
  return w ^ (0x80008000u | (s - (s >> 15)));
}

__device__ __forceinline__ void count_wrap(CountLds& sh, uint32_t k) {
  const uint32_t e = __hip_atomic_fetch_add(&sh.nev, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (e < (uint32_t)kCountEvents) sh.ev[e] = k;
}

// CHECK: the atomic returns the old word, and a counter that was 0xFFFF has
// wrapped (a low one carrying into the high one, which may wrap in turn).
template <bool CHECK>
__device__ __forceinline__ void count_key(CountLds& sh, uint32_t k) {
  const uint32_t inc = (k >> 15) * 0xFFFFu + 1u;
  uint32_t* w = sh.cnt + (k & 0x7FFFu);
  if constexpr (!CHECK) {
    __hip_atomic_fetch_add(w, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else {
    const uint32_t old = __hip_atomic_fetch_add(w, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t lo = old & 0xFFFFu, hi = old >> 16;
    if ((k >> 15) ? hi == 0xFFFFu : lo == 0xFFFFu) {
      count_wrap(sh, k);
      if (!(k >> 15) && hi == 0xFFFFu) count_wrap(sh, k + 32768u);
    }
  }
}
template <bool CHECK>
__device__ __forceinline__ void count_pair(CountLds& sh, uint32_t w) {
  const uint32_t kp = bf16_key_pair(w);
  count_key<CHECK>(sh, kp & 0xFFFFu);
  count_key<CHECK>(sh, kp >> 16);
}

// The counting kernel's layout counts raw bfloat16 bits x (no key
// transform on the hot path): word x & 0x7FFF, the low half for a
// non-negative value, the high half for a negative one.  Raw word w then
// holds key w + 32768 (low) and key 32767 - w (high), which is how the
// finish (finish_list) reads the compacted words.  One add for x: into this lane's
// band copy when x - org < kBandKeys (org a raw origin), else into its
// counter.  blane = 4 (kCountWords + lane): byte offsets.
__device__ __forceinline__ void count_raw(CountLds& sh, uint32_t x, uint32_t org, uint32_t blane) {
  const uint32_t d = x - org;
  const bool in = d < (uint32_t)kBandKeys;
  const uint32_t o = in ? (d << 8) + blane : ((x << 2) & 0x1FFFCu);
  uint32_t* w = static_cast<uint32_t*>(__builtin_assume_aligned(reinterpret_cast<char*>(sh.cnt) + o, 4));
  __hip_atomic_fetch_add(w, ((x >> 15) & 1u) * 0xFFFFu + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void count_pair_raw(CountLds& sh, uint32_t w, uint32_t org, uint32_t blane) {
  count_raw(sh, w & 0xFFFFu, org, blane);
  count_raw(sh, w >> 16, org, blane);
}

// Every logit of the row, once, by threads 0 .. NT - 1.  Lane t takes
// 8-logit units t, t + NT, ... (eight in flight; in the raw layout, batches
// of SV_COUNT_PIPE with the next batch in flight; one in the rarely run
// checked pass, whose code stays small), then one of the last V mod 8.
// RAW: the raw-bit layout of the counting kernel, whose values from the raw
// origin org up go to the band's copies.
template <bool VEC, bool CHECK, int NT, bool RAW = false>
__device__ void count_row(const uint16_t* row, int64_t V, CountLds& sh, uint32_t org = kBandOff) {
  const int t = threadIdx.x;
  const int64_t units = V >> 3;
  int64_t u = t;
  if constexpr (VEC) {
    constexpr int U = CHECK ? 1 : 8;
    constexpr int64_t kBatch = (int64_t)U * NT;
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(row, (int)(units * 16));
    const int voff = t * 16;
    const int64_t nb = units / kBatch;
    const uint32_t blane = 4u * ((uint32_t)kCountWords + (uint32_t)(t & 63));
    auto count4 = [&](const u32x4& w) {
      if constexpr (RAW) {
        count_pair_raw(sh, w.x, org, blane);
        count_pair_raw(sh, w.y, org, blane);
        count_pair_raw(sh, w.z, org, blane);
        count_pair_raw(sh, w.w, org, blane);
      } else {
        count_pair<CHECK>(sh, w.x);
        count_pair<CHECK>(sh, w.y);
        count_pair<CHECK>(sh, w.z);
        count_pair<CHECK>(sh, w.w);
      }
    };
    if constexpr (RAW) {
      // Batches of P loads, the next one in flight while this one is
      // counted.  Past the last batch the loads take an offset outside the
      // buffer's range, which the hardware answers with zeros and no memory
      // access (rather than a branch around them).
      constexpr int P = SV_COUNT_PIPE;
      constexpr int64_t kB = (int64_t)P * NT;
      const int64_t np = units / kB;
      // Two register sets taken in turn, so no copy ties a batch's wait to
      // the previous batch's counting.
      auto load = [&](u32x4* w, int64_t i) {
#pragma unroll
        for (int q = 0; q < P; ++q)
          w[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, i < np ? (int)((i * kB + q * NT) * 16) : (int)(units * 16), 2);
      };
      if (np > 0) {
        u32x4 wa[P], wb[P];
        load(wa, 0);
        // The scheduling barriers keep the compiler from interleaving one
        // set's counting with the other's, which would wait for loads just
        // issued.
        for (int64_t i = 0; i + 1 < np; i += 2) {
          load(wb, i + 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < P; ++q) count4(wa[q]);
          __builtin_amdgcn_sched_barrier(0);
          load(wa, i + 2);   // nothing read after the last pair of an even count
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int q = 0; q < P; ++q) count4(wb[q]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (np & 1) {
#pragma unroll
          for (int q = 0; q < P; ++q) count4(wa[q]);
        }
      }
      u = np * kB + t;
    } else {
      for (int64_t i = 0; i < nb; ++i) {
        u32x4 w[U];
#pragma unroll
        for (int q = 0; q < U; ++q)
          w[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, (int)((i * kBatch + q * NT) * 16), 2);
#pragma unroll
        for (int q = 0; q < U; ++q) count4(w[q]);
      }
      u = nb * kBatch + t;
    }
    for (; u < units; u += NT)
      count4(__builtin_amdgcn_raw_buffer_load_b128(rs, voff, (int)((u - t) * 16), 2));
  } else {
    const uint32_t blane = 4u * ((uint32_t)kCountWords + (uint32_t)(t & 63));
    for (; u < units; u += NT) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t w = (uint32_t)row[u * 8 + e] | ((uint32_t)row[u * 8 + e + 1] << 16);
        if constexpr (RAW) count_pair_raw(sh, w, org, blane);
        else count_pair<CHECK>(sh, w);
      }
    }
  }
  if (t < V - units * 8) {
    const uint32_t x = row[units * 8 + t];
    if constexpr (RAW) count_raw(sh, x, kBandOff, 0u);
    else count_key<CHECK>(sh, bf16_key_pair(x) & 0xFFFFu);
  }
}

// The band's origin for a row of V logits (one wave): a 16-byte load at each
// of 64 evenly spaced places (band_sample), then the 64 values from 32 below
// the lower median of those 512 up, found by a binary search over the key
// range and moved, if they straddle zero, to the median's side (band_origin,
// the same value in every lane).  It returns the band's lowest raw bits:
// keys k .. k + 63 below 32768 (negative values) are raw bits
// 65472 - k .. 65535 - k, keys from 32768 up raw bits k - 32768 on.  Any
// origin counts the row exactly; a good one puts most of its logits in the
// band.  kBandOff for rows shorter than 64 loads or longer than kBandMaxV.
__device__ __forceinline__ bool band_rows(int64_t V) { return V >= 512 && V <= kBandMaxV; }
__device__ __forceinline__ u32x4 band_sample(const uint16_t* row, int64_t V) {
  const int64_t units = V >> 3;
  const int lane = threadIdx.x & 63;
  const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(row, (int)(units * 16));
  return __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(units * lane / 64) * 16, 0, 2);
}
__device__ __forceinline__ uint32_t band_origin(const u32x4& w) {
  uint32_t k[8];
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t kp = bf16_key_pair(x[i]);
    k[2 * i] = kp & 0xFFFFu;
    k[2 * i + 1] = kp >> 16;
  }
  uint32_t lo = 0u, hi = 0xFFFFu;   // the smallest m with at least 256 keys <= m
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    int c = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) c += __popcll(__ballot(k[e] <= mid));
    if (c >= 256) hi = mid;
    else lo = mid + 1u;
  }
  uint32_t ko = min(lo - min(lo, 32u), 0x10000u - (uint32_t)kBandKeys);
  if (ko < 0x8000u && ko + kBandKeys > 0x8000u) ko = lo < 0x8000u ? 0x8000u - kBandKeys : 0x8000u;
  return ko < 0x8000u ? 0xFFC0u - ko : ko - 0x8000u;
}

__device__ __forceinline__ bool key_finite(uint32_t k) { return k > kKeyNegInf && k < kKeyPosInf; }
// Flags of a key outside the finite range: 1 for a NaN, 2 for +inf, 0 for -inf.
__device__ __forceinline__ int nonfinite_flag(uint32_t k) {
  return k == kKeyNegInf ? 0 : (k == kKeyPosInf ? 2 : 1);
}

// The count of key k from its 16-bit counter and the recorded wraps: 65536
// more per wrap of k, one less per carry into k (a wrap of the low counter
// of k's word, when k is the high one).
__device__ __forceinline__ uint32_t key_count(const CountLds& sh, int nev, uint32_t k) {
  uint32_t h = (sh.cnt[k & 0x7FFFu] >> (16 * (k >> 15))) & 0xFFFFu;
  for (int e = 0; e < nev; ++e) {
    const uint32_t x = sh.ev[e];
    if (x == k) h += 65536u;
    else if ((k >> 15) && x == k - 32768u) h -= 1u;
  }
  return h;
}

// Inclusive suffix sum over the lanes of a wave (lane 63 first).
template <typename F>
__device__ __forceinline__ F wave_suffix_sum(F v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const F y = __shfl_down(v, o, 64);
    if (lane + o < 64) v += y;
  }
  return v;
}

// A counted row's outputs: its normaliser piece (the whole row in piece 0,
// -inf in the others) and maximum where the stream items would put them,
// and its nucleus (threshold sel, mass fraction P; none for a bad row).
// Threads tid = 0 .. nthr - 1.
__device__ __forceinline__ void count_outputs(const VerifyArgs& a, int64_t row, int flags, int kmax, float mref,
                                              double Z, int sel, double P, int tid, int nthr) {
  const bool bad = flags != 0 || kmax < 0;
  const float vmax = kmax >= 0 ? key_logit<kBF16>((uint32_t)kmax) : -INFINITY;
  const int64_t p0 = row * a.nc;
  for (int i = tid; i < a.nc; i += nthr) {
    double v = -INFINITY;
    float mr = -INFINITY;
    if (i == 0) {
      if (flags & 1) v = NAN;
      else if (flags & 2) v = INFINITY;
      else if (kmax >= 0) v = (double)mref + log2(Z);
      mr = (flags & 2) ? INFINITY : vmax;
    }
    slot_put32(SV_AT(a, mraw, p0 + i), mr);
    slot_put(SV_AT(a, part, p0 + i), v);
  }
  if (tid == 0) {
    TopPRow tr;
    tr.M = mref;
    tr.Z = Z;
    tr.rem = 0.0;
    tr.above = 0.0;
    const bool cut = !bad && sel >= 0;
    tr.P = cut ? P : 1.0;
    tr.prefix = cut ? (uint32_t)sel : 0u;
    tr.L = cut ? key_logit<kBF16>((uint32_t)sel) : -INFINITY;
    *SV_AT(a, topp, row) = tr;
  }
}

// The in-place finish of a counted row (every thread; topp_redo_kernel):
// wave w takes words 2048w + 64j + lane (j = 0..31), consecutive words in
// consecutive lanes, so a band of crowded values spreads over the lanes.
// From the top key down the order is: the high halves (non-negative values)
// of waves 15..0, then the low halves of waves 15..0; within a wave, rows
// j = 31..0, lanes 63..0.  checked: the counters come from the checked
// pass (its wraps are recorded); otherwise, if they sum to less than V, the
// row is counted again with the checked pass first.  Leaves counts in the
// counters.
template <bool VEC>
__device__ void finish_inplace(const VerifyArgs& a, int64_t row, CountLds& sh, bool checked) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int R = 2 * a.gamma + 1;
  const int b = (int)(row / R), r = (int)(row - (int64_t)b * R);
  const uint16_t* rp = static_cast<const uint16_t*>(row_ptr<kBF16>(a, b, r));
  const TCoef tc = temp_coef(a, b);
  uint4* c4 = reinterpret_cast<uint4*>(sh.cnt);

  // Word of row j: wbase + 64 j (the opaque step keeps the compiler from
  // precomputing every such address outside the caller's loop).
  uint32_t wbase = 2048u * (uint32_t)wave + (uint32_t)lane;
  asm volatile("" : "+v"(wbase));
  // The counter words are read from LDS where used (rare path: registers
  // stay free).
  auto cw = [&](int j) -> uint32_t { return sh.cnt[wbase + 64u * j]; };
  int nev = checked ? (int)min(sh.nev, (uint32_t)kCountEvents) : 0;
  if (!checked) {   // the 16-bit counters sum to V unless one wrapped: then count again, recording the wraps
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) sum += (cw(j) & 0xFFFFu) + (cw(j) >> 16);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    if (lane == 0) sh.sum[wave] = sum;
    __syncthreads();
    sum = 0;
    for (int i = 0; i < kCountWaves; ++i) sum += sh.sum[i];
    if ((int64_t)sum != a.V) {
      __syncthreads();   // every thread is done with the counters
      for (int i = t; i < kCountWords / 4; i += kCountThreads) c4[i] = make_uint4(0u, 0u, 0u, 0u);
      if (t == 0) sh.nev = 0u;
      __syncthreads();
      count_row<VEC, true, kCountThreads>(rp, a.V, sh);
      __syncthreads();
      nev = (int)min(sh.nev, (uint32_t)kCountEvents);
    }
  }
  // The count of key half h of row j (with the recorded wraps, if any); -0
  // counts with +0 (key 0x8000, the high half of word 0).
  const uint32_t nzero = key_count(sh, nev, kKeyNegZero);
  auto count_at = [&](int j, int h) -> uint32_t {
    const uint32_t k = wbase + 64u * j + 32768u * h;
    uint32_t n = nev ? key_count(sh, nev, k) : ((cw(j) >> (16 * h)) & 0xFFFFu);
    return k == kKeyNegZero ? 0u : (k == kKeyPosZero ? n + nzero : n);
  };

  // The largest finite key with a count, and flags (1: a NaN, 2: +inf).
  // Keys outside the finite range: the low halves of words 0..127 (wave 0,
  // rows 0 and 1) and the high halves of words 32640..32767 (wave 15, rows
  // 30 and 31).
  int kmax = -1, flags = 0;
  auto take = [&](uint32_t k, uint32_t n) {
    const bool fin = key_finite(k);
    kmax = (n != 0u && fin) ? max(kmax, (int)k) : kmax;
    flags |= (n != 0u && !fin) ? nonfinite_flag(k) : 0;
  };
  if (nev == 0) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t w = cw(j);
      asm volatile("" : "+v"(w), "+v"(kmax), "+v"(flags));
      const uint32_t k = wbase + 64u * j;
      take(k, k == kKeyNegZero ? 0u : (w & 0xFFFFu));
      take(k + 32768u, k == 0u ? (w >> 16) + nzero : (w >> 16));
    }
  } else {
    for (uint32_t j = 0; j < 32u; ++j)
      for (uint32_t h = 0; h < 2u; ++h) {
        const uint32_t k = wbase + 64u * j + 32768u * h;
        const uint32_t n = key_count(sh, nev, k);
        take(k, k == kKeyNegZero ? 0u : (k == kKeyPosZero ? n + nzero : n));
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmax = max(kmax, __shfl_xor(kmax, o, 64));
    flags |= __shfl_xor(flags, o, 64);
  }
  if (lane == 0) {
    sh.kmax[wave] = kmax;
    sh.flags[wave] = flags;
  }
  __syncthreads();
  for (int i = 0; i < kCountWaves; ++i) {
    kmax = max(kmax, sh.kmax[i]);
    flags |= sh.flags[i];
  }

  // Masses count * 2^(l c_T - mref) (0 for no count or a key outside the
  // finite range): each wave's sums over its high and low halves, in fp64.
  const bool bad = flags != 0 || kmax < 0;
  const float vmax = kmax >= 0 ? key_logit<kBF16>((uint32_t)kmax) : -INFINITY;
  const float mref = bad ? 0.f : ceilf(fminf(vmax * tc.c_hi, 1.0e30f));
  auto mass = [&](uint32_t k, uint32_t n) -> float {
    const float v = key_logit<kBF16>(k);
    const float m = (float)n * exp2_fast(fmaf(v, tc.c_lo, fmaf(v, tc.c_hi, -mref)));
    return (n != 0u && key_finite(k)) ? m : 0.f;
  };
  double cs[2] = {0.0, 0.0};
  if (!bad) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      // One row at a time (the opaque step orders them): computing every
      // term ahead of the additions would not fit the registers.
      uint32_t w = cw(j);
      asm volatile("" : "+v"(w), "+v"(cs[0]), "+v"(cs[1]));
      if (w != 0u || nev != 0 || (t == 0 && j == 0)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) cs[h] += (double)mass(wbase + 64u * j + 32768u * h, count_at(j, h));
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const double wt = wave_sum(cs[h]);
    if (lane == 0) sh.tot[h][wave] = wt;
  }
  if (t == 0) sh.sel = -1;
  __syncthreads();

  // Running sums over the 32 (half, wave) blocks from the top, the same
  // additions in the same order in every thread: Z, and the first block at
  // whose end the sum reaches top_p * Z (ab: the sum before it).
  double Z = 0.0;
  for (int i = 2 * kCountWaves - 1; i >= 0; --i) Z = Z + sh.tot[i / kCountWaves][i % kCountWaves];
  const double tgt = (double)a.top_p * Z;
  double ab = 0.0;
  int hx = -1, wx = -1;
  {
    double run = 0.0;
    for (int i = 2 * kCountWaves - 1; i >= 0 && hx < 0; --i) {
      const double bt = sh.tot[i / kCountWaves][i % kCountWaves], nx = run + bt;
      if (bt > 0.0 && nx >= tgt) {
        hx = i / kCountWaves;
        wx = i % kCountWaves;
        ab = run;
      }
      run = nx;
    }
  }
  if (!bad && wave == wx) {
    // The rows' sums of half hx over the lanes: a butterfly that halves the
    // rows each lane carries at every step leaves row lane / 2 in lanes
    // 2j and 2j + 1.
    float m[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) m[j] = mass(wbase + 64u * j + 32768u * hx, count_at(j, hx));
#pragma unroll
    for (int step = 0; step < 5; ++step) {
      const int half = 16 >> step, o = 32 >> step;
      const bool up = (lane & o) != 0;
#pragma unroll
      for (int k = 0; k < half; ++k) {
        const float send = up ? m[k] : m[k + half];
        const float recv = __shfl_xor(send, o, 64);
        m[k] = (up ? m[k + half] : m[k]) + recv;
      }
    }
    const float rj = m[0] + __shfl_xor(m[0], 1, 64);   // row lane / 2
    // Suffix sums over the rows (row 31 first): lane 2j holds rows >= j.
    const double sj = wave_suffix_sum((lane & 1) ? 0.0 : (double)rj, lane);
    const double incl = ab + sj;
    const double nxt = __shfl_down(sj, 2, 64);
    const double above = lane >= 62 ? ab : ab + nxt;
    const uint64_t crossr = __ballot(!(lane & 1) && rj > 0.f && above < tgt && tgt <= incl);
    const uint64_t hasr = __ballot(!(lane & 1) && rj > 0.f);
    // The crossing row; rounding aside (the rows' sums and the block's
    // differ in order), else the lowest row with mass.
    const int jl = crossr ? (63 - __builtin_clzll(crossr)) : __builtin_ctzll(hasr);
    const int jx = jl >> 1;
    const double ab_row = __shfl(above, jl, 64);
    // Keys of row jx, one per lane: the highest with mass whose running sum
    // reaches the target ends the nucleus (else the lowest with mass).
    const uint32_t k = wbase + 64u * (uint32_t)jx + 32768u * (uint32_t)hx;
    uint32_t n = nev ? key_count(sh, nev, k) : ((sh.cnt[k & 0x7FFFu] >> (16 * hx)) & 0xFFFFu);
    n = k == kKeyNegZero ? 0u : (k == kKeyPosZero ? n + nzero : n);
    const float mk = mass(k, n);
    const double run = wave_suffix_sum((double)mk, lane) + ab_row;
    const uint64_t hit = __ballot(mk != 0.f && run >= tgt);
    const uint64_t has = __ballot(mk != 0.f);
    const int src = hit ? 63 - __builtin_clzll(hit) : __builtin_ctzll(has);
    if (lane == src) {
      sh.sel = (int)k;
      sh.P = run / Z;
    }
  }
  __syncthreads();
  count_outputs(a, row, flags, kmax, mref, Z, sh.sel, sh.P, t, kCountThreads);
}

// The previous row's finish from its compacted raw words (one wave, while
// the other waves count the next row).  Lane l takes a run of consecutive
// entries.  Entry x holds raw value x (non-negative, key x + 32768) in its
// low half and raw value 0x8000 + x (negative, key 32767 - x) in its high
// half, so from the top key down the order is the low halves of entries
// E-1..0, then the high halves of entries 0..E-1.  -0 has been counted with
// +0 already and no counter wrapped.
__device__ void finish_list(const VerifyArgs& a, int64_t row, const CountLds& sh, int E) {
  const int lane = threadIdx.x & 63;
  const int R = 2 * a.gamma + 1;
  const int b = (int)(row / R);
  const TCoef tc = temp_coef(a, b);
  const int per = (E + 63) >> 6;
  const int e0 = min(lane * per, E), e1 = min(e0 + per, E);
  auto key = [](uint32_t x, int h) -> uint32_t { return h ? 0x7FFFu - x : x + 0x8000u; };
  int kmax = -1, flags = 0;
  for (int e = e0; e < e1; ++e) {
    const uint2 en = sh.list[e];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t k = key(en.x, h), n = (en.y >> (16 * h)) & 0xFFFFu;
      if (n == 0u) continue;
      if (key_finite(k)) kmax = max(kmax, (int)k);
      else flags |= nonfinite_flag(k);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmax = max(kmax, __shfl_xor(kmax, o, 64));
    flags |= __shfl_xor(flags, o, 64);
  }
  const bool bad = flags != 0 || kmax < 0;
  const float vmax = kmax >= 0 ? key_logit<kBF16>((uint32_t)kmax) : -INFINITY;
  const float mref = bad ? 0.f : ceilf(fminf(vmax * tc.c_hi, 1.0e30f));
  auto mass = [&](uint32_t k, uint32_t n) -> float {
    const float v = key_logit<kBF16>(k);
    const float m = (float)n * exp2_fast(fmaf(v, tc.c_lo, fmaf(v, tc.c_hi, -mref)));
    return (n != 0u && key_finite(k)) ? m : 0.f;
  };
  double sm[2] = {0.0, 0.0};   // this lane's masses: non-negative values, negative values
  if (!bad) {
    for (int e = e0; e < e1; ++e) {
      const uint2 en = sh.list[e];
      sm[0] += (double)mass(key(en.x, 0), en.y & 0xFFFFu);
      sm[1] += (double)mass(key(en.x, 1), en.y >> 16);
    }
  }
  // Running masses from the top: a suffix sum over the lanes for the
  // non-negative values (lane 63 holds the largest), then, below their total
  // H, a prefix sum for the negative ones (lane 0 holds the largest).  A
  // lane's `above` is the `incl` of the lane before it in that order, taken
  // from that lane (lane 0's negative part starts at H, lane 0's `incl` of
  // the non-negative part), so the intervals tile (0, Z] exactly.
  const double s0 = wave_suffix_sum(sm[0], lane);
  const double p1 = wave_inclusive_scan(sm[1]);
  const double H = __shfl(s0, 0, 64);
  const double d0 = __shfl_down(s0, 1, 64);
  const double incl0 = s0, above0 = lane == 63 ? 0.0 : d0;
  const double incl1 = p1 + H;
  const double u1 = __shfl_up(incl1, 1, 64);
  const double above1 = lane == 0 ? H : u1;
  const double Z = __shfl(incl1, 63, 64);
  const double tgt = (double)a.top_p * Z;
  const bool c0 = !bad && above0 < tgt && tgt <= incl0, c1 = !bad && above1 < tgt && tgt <= incl1;
  int sel = -1;
  double P = 1.0;
  if (c0 || c1) {   // this lane's entries hold the threshold: walk them from the top
    const int h = c0 ? 0 : 1;
    double run = c0 ? above0 : above1, Pl = run;
    int low = -1;
    for (int i = 0; i < e1 - e0; ++i) {
      const int e = h ? e0 + i : e1 - 1 - i;
      const uint2 en = sh.list[e];
      const uint32_t k = key(en.x, h);
      const float m = mass(k, (en.y >> (16 * h)) & 0xFFFFu);
      if (m == 0.f) continue;
      run += (double)m;
      low = (int)k;
      Pl = run;
      if (run >= tgt) break;
    }
    sel = low;
    P = Pl / Z;
  }
  const uint64_t who = __ballot(sel >= 0);
  if (who) {
    const int src = __builtin_ctzll(who);
    sel = __shfl(sel, src, 64);
    P = __shfl(P, src, 64);
  }
  count_outputs(a, row, flags, kmax, mref, Z, sel, P, lane, 64);
}

// Persistent: work-group g counts rows g, g + G, ...  While waves 0..14
// count a row, wave 15 finishes the row before it from its compacted words
// (the counting is limited by LDS atomics, the finish by latency, so they
// overlap).  After each row every thread compacts its words with a count
// into the list and clears its counters; a row whose 16-bit counters
// wrapped, or whose words do not fit the list, is left to topp_redo_kernel
// (keeping the in-place finish out of this kernel keeps its registers).
template <bool VEC>
__global__ __launch_bounds__(kCountThreads) void topp_count_kernel(VerifyArgs, int64_t nrows) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ CountLds sh;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int R = 2 * a.gamma + 1;
  uint4* c4 = reinterpret_cast<uint4*>(sh.cnt);
  for (int i = t; i < (kCountWords + kBandWords) / 4; i += kCountThreads) c4[i] = make_uint4(0u, 0u, 0u, 0u);
  const bool banded = VEC && band_rows(a.V);
  auto rowp = [&](int64_t row) {
    const int b = (int)(row / R), r = (int)(row - (int64_t)b * R);
    return static_cast<const uint16_t*>(row_ptr<kBF16>(a, b, r));
  };
  if (wave == kCountingWaves) {
    const uint32_t o = banded && (int64_t)blockIdx.x < nrows ? band_origin(band_sample(rowp(blockIdx.x), a.V))
                                                             : kBandOff;
    if (lane == 0) sh.org[0] = o;
  }
  __syncthreads();
  int64_t prev = -1;
  int E = 0;
  for (int64_t row = blockIdx.x, n = 0;; row += gridDim.x, ++n) {
    const bool have = row < nrows;
    const uint32_t org = sh.org[n & 1];
    if (wave < kCountingWaves) {
      if (have) count_row<VEC, false, kCountingThreads, true>(rowp(row), a.V, sh, org);
    } else {
      // The next row's sample flies while the previous row is finished.
      const int64_t next = row + gridDim.x;
      const bool s = banded && next < nrows;
      const u32x4 w = s ? band_sample(rowp(next), a.V) : u32x4{0u, 0u, 0u, 0u};
      if (prev >= 0) finish_list(a, prev, sh, E);
      const uint32_t o = s ? band_origin(w) : kBandOff;
      if (lane == 0) sh.org[(n + 1) & 1] = o;
    }
    __syncthreads();
    if (!have) break;

    // The band's copies into the counters: thread t sums copies
    // 4 (t & 15) .. 4 (t & 15) + 3 of raw value org + (t >> 4), clears them,
    // and the value's 16 threads add up; a count that overflows its 16-bit
    // counter leaves the counters' sum short of V, as any wrap does.
    if (org != kBandOff) {
      const uint32_t k = org + (uint32_t)(t >> 4), sh16 = 16u * (k >> 15);
      uint4* bw = reinterpret_cast<uint4*>(sh.cnt + kCountWords) + t;
      const uint4 w = *bw;
      *bw = make_uint4(0u, 0u, 0u, 0u);
      int c = (int)((w.x >> sh16) + (w.y >> sh16) + (w.z >> sh16) + (w.w >> sh16));
      c = row16_reduce(c, [](int x, int y) { return x + y; });
      if ((t & 15) == 0) sh.cnt[k & 0x7FFFu] += (uint32_t)c << sh16;
      __syncthreads();
    }

    // Compaction of the raw words.  -0 (raw 0x8000, the high half of word
    // 0) moves to +0 (raw 0, its low half); the sum of the counters checks
    // for a wrap.  Words are read from LDS as needed (registers stay free
    // for the counting); word of row j: wbase + 64 j.
    uint32_t wbase = 2048u * (uint32_t)wave + (uint32_t)lane;
    asm volatile("" : "+v"(wbase));
    auto word = [&](int j) -> uint32_t {
      uint32_t w = sh.cnt[wbase + 64u * j];
      if (t == 0 && j == 0) w = (w & 0xFFFFu) + (w >> 16);   // checked against overflow below
      return w;
    };
    uint32_t sum = 0, nzc = 0;
    int over = t == 0 && (sh.cnt[0] & 0xFFFFu) + (sh.cnt[0] >> 16) > 0xFFFFu;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const uint32_t w = sh.cnt[wbase + 64u * j];
      sum += (w & 0xFFFFu) + (w >> 16);
      nzc += (uint32_t)__popcll(__ballot(word(j) != 0u));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    over = __ballot(over) != 0;
    if (lane == 0) {
      sh.sum[wave] = sum;
      sh.nzw[wave] = nzc;
      sh.flags[wave] = over;
    }
    __syncthreads();
    uint32_t tsum = 0, base = 0, tot = 0;
    for (int i = 0; i < kCountWaves; ++i) {
      tsum += sh.sum[i];
      base += i < wave ? sh.nzw[i] : 0u;
      tot += sh.nzw[i];
      over |= sh.flags[i];
    }
    if ((int64_t)tsum == a.V && tot <= (uint32_t)kListCap && !over) {
      // Each thread reads only its own words here, so it clears each once
      // read.
      const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll 8
      for (int j = 0; j < 32; ++j) {
        const uint32_t w = word(j);
        sh.cnt[wbase + 64u * j] = 0u;
        const uint64_t bal = __ballot(w != 0u);
        if (w != 0u) sh.list[base + (uint32_t)__popcll(bal & lt)] = make_uint2(wbase + 64u * j, w);
        base += (uint32_t)__popcll(bal);
      }
      prev = row;
      E = (int)tot;
    } else {   // left to topp_redo_kernel
      if (t == 0) {
        const unsigned i = __hip_atomic_fetch_add(SV_AT(a, redo, 0), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const unsigned wrapped = (int64_t)tsum != a.V ? kRedoWrapped : 0u;
        __hip_atomic_store(SV_AT(a, redo, 2 + i), ((unsigned)row + 1u) | wrapped, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      for (int i = t; i < kCountWords / 4; i += kCountThreads) c4[i] = make_uint4(0u, 0u, 0u, 0u);
      prev = -1;
    }
    __syncthreads();
  }
}

// The rows the counting kernel left (16-bit counters that wrapped, or more
// words with a count than its list holds), each counted again - with the
// checked pass straight away where the counters wrapped - and finished in
// place by a whole work-group.  Clears the list as it goes; the last
// work-group to finish clears the two counters.  Launched after the
// counting kernel on the same stream, so the list is complete.
template <bool VEC>
__global__ __launch_bounds__(kCountThreads) void topp_redo_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ CountLds sh;
  const int t = threadIdx.x;
  const unsigned n = __hip_atomic_load(SV_AT(a, redo, 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  uint4* c4 = reinterpret_cast<uint4*>(sh.cnt);
  for (unsigned i = blockIdx.x; i < n; i += gridDim.x) {
    const unsigned e = __hip_atomic_load(SV_AT(a, redo, 2 + i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int64_t row = SV_IDX(a, (int64_t)(e & ~kRedoWrapped) - 1, (int64_t)a.B * (2 * a.gamma + 1));
    const bool wrapped = (e & kRedoWrapped) != 0u;
    for (int j = t; j < kCountWords / 4; j += kCountThreads) c4[j] = make_uint4(0u, 0u, 0u, 0u);
    if (t == 0) sh.nev = 0u;
    __syncthreads();
    const int R = 2 * a.gamma + 1;
    const int b = (int)(row / R), r = (int)(row - (int64_t)b * R);
    const uint16_t* rp = static_cast<const uint16_t*>(row_ptr<kBF16>(a, b, r));
    if (wrapped) count_row<VEC, true, kCountThreads>(rp, a.V, sh);   // record the wraps at once
    else count_row<VEC, false, kCountThreads>(rp, a.V, sh);
    __syncthreads();
    finish_inplace<VEC>(a, row, sh, wrapped);
    __syncthreads();
    if (t == 0) __hip_atomic_store(SV_AT(a, redo, 2 + i), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (t == 0) {
    const unsigned d = __hip_atomic_fetch_add(SV_AT(a, redo, 1), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (d == gridDim.x - 1) {
      __hip_atomic_store(SV_AT(a, redo, 0), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(SV_AT(a, redo, 1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace sv
