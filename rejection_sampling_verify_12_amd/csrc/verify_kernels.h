// Kernels: the single kernel and one kernel per item kind.
#pragma once
#include "verify_sched.h"

#undef SV_FILE
#define SV_FILE 6

namespace sv {

// ---------------------------------------------------------------------------
// Kernels.

#ifndef SV_TIMELINE
#define SV_TIMELINE 0
#endif
#if SV_TIMELINE
// Measurement build only: per block of the single kernel, its start and end
// (s_memrealtime, 100 MHz), item (kind | sub << 8), sequence, and the
// hardware ids of the CU and XCC it ran on.  Read with spec_timeline_copy.
constexpr unsigned kTimelineBlocks = 1u << 17;
__device__ uint4 g_timeline[2 * kTimelineBlocks];
#endif

union ItemLds {
  StreamLds s;
  DecideLds d;
  DrawLds r;
  FinalLds f;
  TestLds t;
};

// Early exit: a stream item of position pos (1..gamma-1) skips its rows when
// an earlier position is known to stop the sequence; an item of target row
// gamma (pos = gamma) skips on any known stop.  Read by one thread; the
// work-group follows its answer.
__device__ __forceinline__ bool early_stopped(const VerifyArgs& a, int b, int pos) {
  const unsigned st = ld_dev_u32(SV_AT(a, flag, (int64_t)b * kFlagStride + kStopWord));
  return pos >= a.gamma ? st != 0u : st > 64u - (unsigned)pos;
}
// A skipping item publishes skip markers in place of its piece.
__device__ __forceinline__ void early_skip(const VerifyArgs& a, int b, int r, int c) {
  if (threadIdx.x == 0) {
    const int64_t idx = ((int64_t)b * (2 * a.gamma + 1) + r) * a.nc + c;
    __hip_atomic_store(SV_AT(a, mraw, idx), kSkipRaw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    st_dev_u64(SV_AT(a, part, idx), kSkipPiece);
  }
}

// Packed bf16 rows: compiled for 8 waves per SIMD (64 VGPRs), which the
// stream items need; only the refined draw spills (a few registers, on its
// own path).  float32 and unaligned rows hold twice the registers per logit
// in flight, and their sampling paths need more: 4 waves per SIMD (128 VGPRs).
template <int DT, bool VEC>
constexpr int kFusedWaves = DT == kBF16 && VEC ? 8 : 4;

// The single kernel's one argument: the call and its launch order.
struct FusedArgs {
  VerifyArgs a;
  Sched sc;
};

// PRED: outcome prediction too (draft-row items record lane leaders; the
// items of target row gamma are followed by leader items of draft row gamma).
// EARLY: the early-exit order (position-major stream items, position tests).
// N: tiles per sampling item.
template <int DT, bool VEC, int U, bool PRED, bool EARLY, int N = kTilesPerItem>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFusedWaves<DT, VEC>, 8)))
void fused_kernel(FusedArgs) {
  const FusedArgs& fa = kernel_arg0<FusedArgs>();
  const VerifyArgs& a = fa.a;
  __shared__ ItemLds sh;
  __shared__ int item[4];
#if SV_TIMELINE
  const uint64_t tl_start = __builtin_amdgcn_s_memrealtime();
#endif
  // One wave decodes the block number (a search on the scalar unit, which
  // the CU's waves share) and hands the item to the others.
  if (threadIdx.x < 64) {
    int kind, b, sub;
    // The order is read where the argument segment holds it, with dynamic
    // indices (scalar loads).
    sched_decode_mem(fa.sc, (int)blockIdx.x, kind, b, sub);
    if (threadIdx.x == 0) {
      item[0] = kind;
      item[1] = b;
      item[2] = sub;
      bool skip = false;
      if constexpr (EARLY) {
        if (kind == kItemStream && b >= a.B) skip = early_stopped(a, b - b / a.B * a.B, b / a.B);
        else if (kind == kItemLast) skip = early_stopped(a, b, a.gamma);
      }
      item[3] = skip;
    }
  }
  __syncthreads();
  const int kind = uni(item[0]), b = uni(item[1]), sub = uni(item[2]), skip = uni(item[3]);
#if SV_CHECKS
  // The decoded item: a kind with instances, instance and part in range.
  if (threadIdx.x == 0) {
    const int kd = (int)SV_IDX(a, kind, kKinds);
    SV_IDX(a, b, fa.sc.count[kd]);
    SV_IDX(a, sub, fa.sc.size[kd]);
  }
#endif
  switch (kind) {
    case kItemStream: {
      if constexpr (EARLY) {   // b = i * B + sequence; sub: draft row i, then target row i
        const int i = b / a.B, q = b - i * a.B;
        const int h = sub >= a.nc, c = sub - h * a.nc, r = h ? a.gamma + i : i;
        if (skip) early_skip(a, q, r, c);
        else stream_item<DT, VEC, U>(a, q, r, c, sh.s);
      } else {
        const int r = sub / a.nc, c = sub - r * a.nc;
        if (PRED && r < a.gamma) stream_item<DT, VEC, U, PRED>(a, b, r, c, sh.s);
        else stream_item<DT, VEC, U>(a, b, r, c, sh.s);
      }
      break;
    }
    case kItemTest:
      if constexpr (EARLY) test_item<DT>(a, b - b / a.B * a.B, b / a.B, sh.t);
      break;
    case kItemDecide: decide_item<DT>(a, b, sh.d); break;
    case kItemMass: break;   // Saguaro with eps > 0 runs as separate kernels
    case kItemSample: sample_item<DT, VEC, false, false, N>(a, b, sub, sh.r.lds_d); break;
    case kItemDraw: draw_item<DT, VEC, false, false>(a, b, sh.r); break;
    case kItemLast:
      if (EARLY && skip) {
        early_skip(a, b, 2 * a.gamma, sub);
        break;
      }
      if (!PRED || sub < a.nc) stream_item<DT, VEC, U>(a, b, 2 * a.gamma, sub, sh.s);
      else leader_item<DT, VEC, U>(a, b, sub - a.nc, sh.s);
      break;
    default: final_item<DT, true>(a, b, sh.f); break;
  }
#if SV_TIMELINE
  if (threadIdx.x == 0 && blockIdx.x < kTimelineBlocks) {
    const uint64_t tl_end = __builtin_amdgcn_s_memrealtime();
    unsigned hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    g_timeline[2 * blockIdx.x] = make_uint4((unsigned)tl_start, (unsigned)tl_end,
                                            (unsigned)kind | ((unsigned)sub << 8), (unsigned)b);
    g_timeline[2 * blockIdx.x + 1] = make_uint4(hw, xcc, 0u, 0u);
  }
#endif
}

template <int DT, bool VEC, int U>
__global__ __launch_bounds__(kThreads) void stream_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ StreamLds sh;
  const int R = 2 * a.gamma + 1;
  const int64_t id = blockIdx.x;
  const int per_seq = R * a.nc;
  const int b = (int)(id / per_seq);
  const int rem = (int)(id - (int64_t)b * per_seq);
  const int r = rem / a.nc, c = rem - r * a.nc;
  stream_item<DT, VEC, U>(a, b, r, c, sh);
}

template <int DT, bool CUT>
__global__ __launch_bounds__(kThreads) void decide_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ DecideLds sh;
  decide_item<DT, CUT>(a, blockIdx.x, sh);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void test_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ TestLds sh;
  const int i = blockIdx.x / a.B;
  test_item<DT>(a, blockIdx.x - i * a.B, i, sh);
}

// N tiles per item (a.nt items per sequence).
template <int DT, bool VEC, bool CUT, int N = kTilesPerItem>
__global__ __launch_bounds__(kThreads) void mass_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ double lds_d[kWaves * (kTilesPerItem + 1)];
  const int b = blockIdx.x / a.nt, s = blockIdx.x - b * a.nt;
  mass_item<DT, VEC, CUT, N>(a, b, s, lds_d);
}

// EPS: the call may use the Saguaro eps mode (its weights need more
// registers); N tiles per item (a.nt items per sequence).
template <int DT, bool VEC, bool CUT, bool EPS, int N = kTilesPerItem>
__global__ __launch_bounds__(kThreads) void sample_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ double lds_d[kWaves * (kTilesPerItem + 1)];
  const int b = blockIdx.x / a.nt, s = blockIdx.x - b * a.nt;
  sample_item<DT, VEC, CUT, EPS, N>(a, b, s, lds_d);
}

// The draw and the final item of sequence blockIdx.x, which refines a
// small-residual draw in place: one launch where three would follow the
// sampling.
template <int DT, bool VEC, bool CUT>
__global__ __launch_bounds__(kThreads) void draw_final_kernel(VerifyArgs) {
  const VerifyArgs& a = kernel_arg0<VerifyArgs>();
  __shared__ FinalLds sh;
  draw_item<DT, VEC, CUT>(a, blockIdx.x, sh.r);
  __syncthreads();
  final_item<DT, true, CUT>(a, blockIdx.x, sh);
}

// Zero n 16-byte words (a kernel, not a memset, so a captured call records
// no memset node).
__global__ __launch_bounds__(kThreads) void zero_kernel(uint4* p, size_t n) {
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads) p[i] = z;
}

}  // namespace sv
