// Batched speculative-sampling verification for gfx950.
//
// The rule is the one of "Speculative Decoding: small model guesses, large
// model verifies" (section 3: accept x iff u < min(1, q(x)/p(x)), stop at the
// first rejection, resample from (q-p)+ / sum(q-p)+; section 2: the bonus
// after gamma acceptances comes from the target's position gamma), with the
// Saguaro resampling option of "Speculative Speculative Decoding (Saguaro)"
// (section 3.2: proportional to sqrt(p_D * p_residual)).
//
// Work items (each one 256-thread work-group's job):
//   stream (b, r, c): stream chunk c of row r of sequence b once from HBM and
//     reduce it to a piece of the row's tempered-softmax log-normaliser,
//     v = log2 sum_j 2^(l_j c_T), c_T = log2(e) / T.  c_T is an unevaluated
//     float pair (two FMAs per logit) so the temperature is exact; each lane
//     keeps an integer offset, so every rescale is an exact ldexp, tree-sums
//     each batch of its logits in fp32 and accumulates in fp64.
//   decide (b): merge the pieces of the rows the accept tests read (fp64),
//     run the accept test at every draft position (fp64, wave ballot -> first
//     rejection k) and write the sequence's decision record.
//   residual mass (b, s), Saguaro with eps > 0 only: the residual weight sum
//     over a few 2048-logit tiles of row pair k, which the eps clamp needs.
//   sample (b, s): per-tile sums of the sampling weights over a few tiles of
//     row pair k, or of target row gamma after a full acceptance (the bonus
//     draw, each tile with its own offset, so it needs no row normaliser).
//   draw (b): locate the tile holding u * total (fp64 scan over the tile
//     sums, token order) and rescan it (fp64 prefix over the same per-lane
//     fp32 sums): the drawn token.
//   final (b): check target row gamma (read by the bonus draw only, hence
//     streamed last) and write the outputs.
//
// Hand-off between work-groups uses 64-bit slots that are 0 when empty: a
// producer stores ~bits(value) with one device-coherent store, a consumer
// polls (bounded) until the slot is nonzero and clears it after use, so the
// workspace is all zero again when a call ends.  No item waits for anything
// but items of the same sequence that come earlier in the launch order.
//
// Default launch: one kernel whose blocks run the items in steps (the
// launch order, verify_sched.h): the stream items of sequence t, then the
// later items of earlier sequences, so that a sequence's decision, sampling
// and draw run while other sequences stream; the target rows gamma, which
// no decision waits for, come last.  Work-groups are dispatched in block order, so the
// smallest unfinished block has every item it waits for finished and can
// always run; a wait that still times out sets the error word and gives up
// instead of hanging.
//
// Device code, in include order: verify_args.h (arguments, slots, helpers),
// verify_stream.h, verify_decide.h (decision and early-exit test items),
// verify_sample.h (sampling weights, mass, sampling, draw and final items),
// verify_sched.h (launch order), verify_kernels.h, verify_topp.h.  This file
// holds the host side: workspace layout, launches and the C entry points.
#include "verify_topp.h"

#include <cmath>
#include <limits.h>
#include <algorithm>
#include <atomic>
#include <mutex>

namespace sv {

// ---------------------------------------------------------------------------
// Host side.

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  int nc, chunk, ntile, nt, nt_max;
  size_t nrec, nrec_d;   // per-chunk records: all rows, draft rows (lane leaders)
  size_t err_off, part_off, mraw_off, seq_off, flag_off, tiles_off, mass_off, rsum_off, cpart_off,
      ref_off, topp_off, hist_off, redo_off, total;
};

static bool sizes_ok(int B, int gamma, int V) { return sizes_in_range(B, gamma, V); }

static Layout layout(int B, int gamma, int V) {
  Layout L;
  // Chunks are a multiple of the batch stride (SV_STREAM_UNROLL * 2048 logits),
  // so only a row's last chunk has a partial batch.  A call with few rows
  // takes shorter chunks (down to kSmallChunk, one tile), so that its rows
  // still spread over many work-groups and each one's loads run fewer batches
  // deep: at one tile a lane issues a single load.  (B=1, gamma=4, V=32000,
  // float32: 22.5 us with chunks of one batch stride, 20.3 us with one tile.)
  const int64_t rows = (int64_t)B * (2 * gamma + 1);
  L.chunk = kChunk;
  while (L.chunk > kSmallChunk && rows * (((int64_t)V + L.chunk - 1) / L.chunk) < kSmallCallItems) L.chunk /= 2;
  L.nc = (int)(((int64_t)V + L.chunk - 1) / L.chunk);
  // Per-chunk records: at least what any call with shortened chunks needs,
  // so that a workspace sized for a call serves every smaller one.
  const size_t nrec = std::max<size_t>((size_t)rows * L.nc, (size_t)kSmallCallItems * (kChunk / kSmallChunk));
  const size_t nrec_d = std::max<size_t>((size_t)B * (gamma + 1) * L.nc, (size_t)kSmallCallItems * (kChunk / kSmallChunk));
  L.nrec = nrec;
  L.nrec_d = nrec_d;
  L.ntile = (V + kTile - 1) / kTile;
  L.nt = (L.ntile + kTilesPerItem - 1) / kTilesPerItem;
  L.nt_max = (L.ntile + kShortTiles - 1) / kShortTiles;   // short calls' sampling items
  const size_t R = 2 * (size_t)gamma + 1;
  size_t off = 0;
  L.err_off = off;
  off += 256;
  L.part_off = off;
  off += align256(nrec * sizeof(uint64_t));
  L.mraw_off = off;
  off += align256(nrec * sizeof(unsigned));
  L.seq_off = off;
  off += align256((size_t)B * sizeof(SeqRec));
  L.flag_off = off;
  off += align256((size_t)B * kFlagStride * sizeof(unsigned));
  L.tiles_off = off;
  off += align256((size_t)B * L.ntile * sizeof(uint64_t));
  L.mass_off = off;
  off += align256((size_t)B * L.nt_max * sizeof(uint64_t));
  L.rsum_off = off;
  off += align256((size_t)B * L.nt_max * sizeof(uint64_t));
  L.cpart_off = off;
  off += align256(nrec_d * sizeof(Top3));
  L.ref_off = off;
  off += align256((size_t)B * L.ntile * 4 * sizeof(uint64_t));
  L.topp_off = off;
  off += align256((size_t)B * R * sizeof(TopPRow));
  L.hist_off = off;
  off += align256((size_t)B * R * kDigits * sizeof(double));
  L.redo_off = off;
  off += align256(((size_t)B * R + 2) * sizeof(unsigned));
  L.total = B == 0 ? 0 : off;
  return L;
}

// Work-groups of the fused kernel the device holds at once, cached per
// device and kernel variant.  The entries are atomics: concurrent callers may
// fill one at the same time, with the same value.
template <int DT, bool VEC, bool PRED, bool EARLY, int N = kTilesPerItem>
static hipError_t resident_groups(int& slots) {
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
        &per_cu, reinterpret_cast<const void*>(fused_kernel<DT, VEC, SV_STREAM_UNROLL, PRED, EARLY, N>),
        kThreads, 0);
  if (e != hipSuccess) return e;
  slots = std::max(1, ncu * per_cu);
  if (c) c->store(slots, std::memory_order_relaxed);
  return hipSuccess;
}

template <int DT, bool VEC>
static hipError_t launch_kernels(const VerifyArgs& a, hipStream_t st);

// Short calls - stream items at most 1.5 times the fused kernel's slots -
// take sampling items of kShortTiles tiles: twice as many, each reading half
// as much, so the last sequences' sampling ends sooner.  Longer calls keep
// kTilesPerItem, whose fewer items leave more slots to the stream while they
// wait.  (B=64, gamma=5, V=128256: 53.7 against 55.7 us; B=128, gamma=4:
// 76.0 against 73.1 us with two tiles.)
static bool short_sampling(const VerifyArgs& a, int slots) {
  return (int64_t)a.B * (2 * a.gamma + 1) * a.nc * 2 <= 3 * (int64_t)slots;
}

// The single kernel with short sampling items (no prediction, no eps, no
// early exit): its own slot count, nt items of kShortTiles tiles.
template <int DT, bool VEC>
static hipError_t launch_short(const VerifyArgs& a, hipStream_t st) {
  int slots = 0;
  hipError_t e = resident_groups<DT, VEC, false, false, kShortTiles>(slots);
  if (e != hipSuccess) return e;
  VerifyArgs b = a;
  b.nt = (a.ntile + kShortTiles - 1) / kShortTiles;
  const Sched sc = make_sched(b.B, 2 * b.gamma * b.nc, b.nc, 0, b.nt, slots);
  hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, false, false, kShortTiles>),
                     dim3((unsigned)sc.total), dim3(kThreads), 0, st, FusedArgs{b, sc});
  return hipGetLastError();
}

// pa: NULL, or outcome prediction after the verification.
template <int DT, bool VEC>
static hipError_t launch_all(const VerifyArgs& a, const PredictArgs* pa, hipStream_t st) {
  // The single-kernel order for packed bf16 rows.  float32 or unaligned rows
  // take it for the plain rule (at half the occupancy, below); with a cut,
  // eps, early exit or prediction they take one kernel per item kind and the
  // stand-alone prediction.
  if constexpr (SV_FUSED && DT == kBF16 && VEC) {
    if (!a.topp && !(a.saguaro && a.eps > 0.f)) {
      int slots = 0;
      const bool eps_mode = a.saguaro && a.eps > 0.f;
      if (a.early) {
        hipError_t e = resident_groups<DT, VEC, false, true>(slots);
        if (e != hipSuccess) return e;
        static_assert(SV_EARLY_CHUNK % SV_CHUNK == 0, "early-exit chunks are whole default chunks");
        VerifyArgs b = a;   // never more chunks than the workspace holds
        b.chunk = a.chunk < kChunk ? a.chunk : SV_EARLY_CHUNK;   // a short call keeps its short chunks
        b.nc = (int)(((int64_t)a.V + b.chunk - 1) / b.chunk);
        const Sched sc = make_sched_early(b.B, b.gamma, b.nc, eps_mode ? b.nt : 0, b.nt, slots);
        hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, false, true>), dim3((unsigned)sc.total),
                           dim3(kThreads), 0, st, FusedArgs{b, sc});
        return hipGetLastError();   // the single kernel's final items refine in place
      }
      hipError_t e = pa ? resident_groups<DT, VEC, true, false>(slots) : resident_groups<DT, VEC, false, false>(slots);
      if (e != hipSuccess) return e;
      if (!pa && short_sampling(a, slots)) return launch_short<DT, VEC>(a, st);
      const Sched sc = make_sched(a.B, 2 * a.gamma * a.nc, (pa ? 2 : 1) * a.nc, eps_mode ? a.nt : 0, a.nt, slots);
      if (pa) {
        hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, true, false>), dim3((unsigned)sc.total),
                           dim3(kThreads), 0, st, FusedArgs{a, sc});
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return predict_launch_leaders(*pa, SPEC_BF16, st);
      }
      hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, false, false>), dim3((unsigned)sc.total),
                         dim3(kThreads), 0, st, FusedArgs{a, sc});
      return hipGetLastError();
    }
  }
  if constexpr (SV_FUSED && !(DT == kBF16 && VEC)) {
    // float32 or unaligned rows: the single kernel in the default order, for
    // the rule without a cut, eps or prediction (one launch instead of a
    // chain of five, which is what a small batch waits for).
    if (!a.topp && !(a.saguaro && a.eps > 0.f) && !a.early && !pa) {
      int slots = 0;
      hipError_t e = resident_groups<DT, VEC, false, false>(slots);
      if (e != hipSuccess) return e;
      if (short_sampling(a, slots)) return launch_short<DT, VEC>(a, st);   // refines in place too
      const Sched sc = make_sched(a.B, 2 * a.gamma * a.nc, a.nc, 0, a.nt, slots);
      hipLaunchKernelGGL((fused_kernel<DT, VEC, SV_STREAM_UNROLL, false, false>), dim3((unsigned)sc.total),
                         dim3(kThreads), 0, st, FusedArgs{a, sc});
      return hipGetLastError();   // its final items refine in place (registers to spare)
    }
  }
  {
    hipError_t e = launch_kernels<DT, VEC>(a, st);
    if (e != hipSuccess || !pa) return e;
    return predict_launch_rows(*pa, DT == kBF16 ? SPEC_BF16 : SPEC_F32, VEC, st);
  }
}

template <int DT, bool VEC, bool CUT>
static hipError_t launch_kernels_cut(const VerifyArgs& a0, hipStream_t st) {
  const int R = 2 * a0.gamma + 1;
  const bool eps_mode = a0.saguaro && a0.eps > 0.f;
  // Saguaro eps on bfloat16 rows without a cut: residual-mass and sampling
  // items of kShortTiles tiles, twice as many (B=256, gamma=8, V=152064:
  // 295.7 against 301.7 us; with a top-p cut the longer items are faster).
  constexpr bool kShortEps = DT == kBF16 && !CUT;
  VerifyArgs a = a0;
  if (kShortEps && eps_mode) a.nt = (a.ntile + kShortTiles - 1) / kShortTiles;
  const unsigned nstream = (unsigned)((int64_t)a.B * R * a.nc);
  const unsigned nsample = (unsigned)((int64_t)a.B * a.nt);
  const unsigned rows = (unsigned)((int64_t)a.B * R);
  if (CUT && DT == kBF16 && a.V <= kCountMaxV) {
    // Counting gives each row's nucleus and its normaliser piece in one read.
    int ncu = 0, dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const unsigned grid = std::min<unsigned>(rows, (unsigned)std::max(ncu, 1));
    hipLaunchKernelGGL((topp_count_kernel<VEC>), dim3(grid), dim3(kCountThreads), 0, st, a, (int64_t)rows);
    // Few work-groups: the rows it redoes are rare, and an empty pass is short.
    hipLaunchKernelGGL((topp_redo_kernel<VEC>), dim3(std::min(grid, 32u)), dim3(kCountThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((stream_kernel<DT, VEC, SV_STREAM_UNROLL>), dim3(nstream), dim3(kThreads), 0, st, a);
    if constexpr (CUT) {   // the nucleus of every row by radix selection
      constexpr int npass = DT == kBF16 ? 2 : 4;
      hipLaunchKernelGGL(topp_init_kernel, dim3(rows), dim3(64), 0, st, a);
      for (int pass = 0; pass < npass; ++pass) {
        hipLaunchKernelGGL((topp_hist_kernel<DT, VEC>), dim3(nstream), dim3(kThreads), 0, st, a, pass);
        hipLaunchKernelGGL((topp_select_kernel<DT>), dim3(rows), dim3(64), 0, st, a, pass, npass);
      }
    }
  }
  if (a.early)   // position-major: the test of (i - 1, b) has a smaller block number than (i, b)'s
    hipLaunchKernelGGL((test_kernel<DT>), dim3((unsigned)((int64_t)a.gamma * a.B)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((decide_kernel<DT, CUT>), dim3((unsigned)a.B), dim3(kThreads), 0, st, a);
  if (kShortEps && eps_mode) {
    hipLaunchKernelGGL((mass_kernel<DT, VEC, CUT, kShortTiles>), dim3(nsample), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL((sample_kernel<DT, VEC, CUT, true, kShortTiles>), dim3(nsample), dim3(kThreads), 0, st, a);
  } else if (eps_mode) {
    hipLaunchKernelGGL((mass_kernel<DT, VEC, CUT>), dim3(nsample), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL((sample_kernel<DT, VEC, CUT, true>), dim3(nsample), dim3(kThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((sample_kernel<DT, VEC, CUT, false>), dim3(nsample), dim3(kThreads), 0, st, a);
  }
  hipLaunchKernelGGL((draw_final_kernel<DT, VEC, CUT>), dim3((unsigned)a.B), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int DT, bool VEC>
static hipError_t launch_kernels(const VerifyArgs& a, hipStream_t st) {
  return a.topp ? launch_kernels_cut<DT, VEC, true>(a, st) : launch_kernels_cut<DT, VEC, false>(a, st);
}

static int verify_impl(const void* draft, const void* target, int dtype, const int32_t* tokens,
                       const float* u_acc, const float* u_smp, int B, int gamma, int V, float T,
                       const int32_t* in_len, int32_t* out_tokens, int32_t* out_acc,
                       int32_t* out_fr, uint64_t* out_mask, int32_t* out_len,
                       const spec_diag* diag, void* ws, size_t ws_bytes, void* stream,
                       int saguaro, float eps, int32_t* cand = nullptr, int32_t* hit = nullptr,
                       int32_t* cand_idx = nullptr, int early = 0, const float* temps = nullptr,
                       float top_p = 1.f) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (!sizes_ok(B, gamma, V)) return SPEC_EINVAL;
  if (!temps && (!(T > 0.f) || !std::isfinite(T))) return SPEC_EINVAL;
  if (temps) T = 1.f;   // unused: every sequence has its own
  if (!(eps >= 0.f) || !std::isfinite(eps)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  if (!draft || !target || !tokens || !u_acc || !u_smp || !out_tokens || !out_acc)
    return SPEC_EINVAL;
  const Layout L = layout(B, gamma, V);
  // Every launch (and the fused kernel's item count) stays within one grid
  // dimension of 2^32 - 1 work-items, with block numbers below 2^31.
  const int64_t items = (int64_t)B * ((2 * gamma + 2) * L.nc + 2 * L.nt_max + 3 + gamma);
  if (items * kThreads > (int64_t)UINT_MAX || items > (int64_t)INT_MAX) return SPEC_EINVAL;
  if (!ws || ws_bytes < L.total) return SPEC_EWORKSPACE;

  VerifyArgs a;
  a.draft = draft;
  a.target = target;
  a.tokens = tokens;
  a.u_acc = u_acc;
  a.u_smp = u_smp;
  a.in_len = in_len;
  a.out_tokens = out_tokens;
  a.out_acc = out_acc;
  a.out_first_reject = out_fr;
  a.out_mask = out_mask;
  a.out_len = out_len;
  if (diag) a.diag = *diag;
  else a.diag = spec_diag{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  char* w = static_cast<char*>(ws);
  a.err = reinterpret_cast<unsigned*>(w + L.err_off);
  a.part = reinterpret_cast<uint64_t*>(w + L.part_off);
  a.mraw = reinterpret_cast<unsigned*>(w + L.mraw_off);
  a.seq = reinterpret_cast<SeqRec*>(w + L.seq_off);
  a.flag = reinterpret_cast<unsigned*>(w + L.flag_off);
  a.tiles = reinterpret_cast<uint64_t*>(w + L.tiles_off);
  a.mass = reinterpret_cast<uint64_t*>(w + L.mass_off);
  a.rsum = reinterpret_cast<uint64_t*>(w + L.rsum_off);
  a.cpart = reinterpret_cast<Top3*>(w + L.cpart_off);
  a.ref = reinterpret_cast<uint64_t*>(w + L.ref_off);
  // Residual draws of a small residual mass are refined in fp64 by a kernel
  // after the call's others.  (A Saguaro call falls back to the residual only
  // on degenerate inputs, and draws that fallback in fp32.)
  a.refine = saguaro ? 0 : 1;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.nc = L.nc;
  a.chunk = L.chunk;
  a.ntile = L.ntile;
  a.nt = L.nt;
  {
    // c_hi is rounded toward zero so that c_lo > 0: a -inf logit then gives
    // fma(-inf, c_lo, -inf) = -inf, never NaN.
    const double c = 1.4426950408889634073599246810019 / (double)T;
    float ch = (float)c;
    if ((double)ch >= c) ch = std::nextafter(ch, 0.f);
    a.c_hi = ch;
    a.c_lo = (float)(c - (double)ch);
    if (!(a.c_lo > 0.f)) a.c_lo = 1.17549435e-38f;
    a.cTd = (double)a.c_hi + (double)a.c_lo;
    a.invT = 1.0 / (double)T;
  }
  a.saguaro = saguaro;
  a.eps = eps;
  a.early = early;
  a.temps = temps;
  a.top_p = top_p;
  a.topp = nullptr;
  a.hist = nullptr;
  a.redo = nullptr;
  if (top_p < 1.f) {
    a.topp = reinterpret_cast<TopPRow*>(w + L.topp_off);
    a.hist = reinterpret_cast<double*>(w + L.hist_off);
    a.redo = reinterpret_cast<unsigned*>(w + L.redo_off);
  }
#if SV_CHECKS
  {
    const int64_t b = B, R = 2 * (int64_t)gamma + 1, cut = a.topp ? 1 : 0;
    a.chk = a.err + 1;
    a.n_part = a.n_mraw = (int64_t)L.nrec;
    a.n_cpart = (int64_t)L.nrec_d;
    a.n_seq = b;
    a.n_flag = b * kFlagStride;
    a.n_tiles = b * L.ntile;
    a.n_mass = a.n_rsum = b * L.nt_max;
    a.n_ref = b * L.ntile * 4;
    a.n_topp = cut * b * R;
    a.n_hist = cut * b * R * kDigits;
    a.n_redo = cut * (b * R + 2);
    a.n_tokens = a.n_u_acc = b * gamma;
    a.n_u_smp = a.n_out_tokens = b * (gamma + 1);
    a.n_in_len = in_len ? b : 0;
    a.n_temps = temps ? b : 0;
    a.n_out_acc = b;
    a.n_out_first_reject = out_fr ? b : 0;
    a.n_out_mask = out_mask ? b : 0;
    a.n_out_len = out_len ? b : 0;
  }
#endif

  PredictArgs p;
  if (cand) {
    p.draft = draft;
    p.accepted = out_acc;
    p.out_tokens = out_tokens;
    p.cand = cand;
    p.hit = hit;
    p.cand_idx = cand_idx;
    p.part = a.cpart;
    p.B = B;
    p.gamma = gamma;
    p.V = V;
    p.nc = L.nc;
    p.chunk = L.chunk;
  }
  const PredictArgs* pa = cand ? &p : nullptr;
  const bool vec = (V % 8 == 0) && ((uintptr_t)draft % 16 == 0) && ((uintptr_t)target % 16 == 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipError_t e;
  if (dtype == SPEC_BF16) e = vec ? launch_all<kBF16, true>(a, pa, st) : launch_all<kBF16, false>(a, pa, st);
  else e = vec ? launch_all<kF32, true>(a, pa, st) : launch_all<kF32, false>(a, pa, st);
  return e == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

// ---------------------------------------------------------------------------
// The allocation-free entry point's workspace: one array per device, in the
// library's own device memory (it lives until the process ends).  Host code
// uses only its device address from hipGetSymbolAddress, fetched once per
// device with that device current.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::atomic<void*> g_scratch_ptr[64];
static std::mutex g_scratch_mu;

static hipError_t scratch_address(void*& ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return hipSuccess;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!p) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  ptr = p;
  return hipSuccess;
}

}  // namespace sv

extern "C" {

size_t spec_workspace_bytes(int B, int gamma, int V, int dtype) {
  if ((dtype != SPEC_F32 && dtype != SPEC_BF16) || !sv::sizes_ok(B, gamma, V)) return 0;
  return sv::layout(B, gamma, V).total;
}

int spec_verify(const void* draft_logits, const void* target_logits, int dtype,
                const int32_t* draft_tokens, const float* u_accept, const float* u_sample, int B,
                int gamma, int V, float temperature, const int32_t* in_len, int32_t* out_tokens,
                int32_t* out_accepted, int32_t* out_first_reject, uint64_t* out_accept_mask,
                int32_t* out_len, const spec_diag* diag, void* workspace, size_t workspace_bytes,
                void* stream) {
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, 0, 0.f);
}

int spec_verify_saguaro(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        int B, int gamma, int V, float temperature, const int32_t* in_len,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                        uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                        void* workspace, size_t workspace_bytes, void* stream, float eps) {
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, 1, eps);
}

int spec_verify_predict(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        int B, int gamma, int V, float temperature, const int32_t* in_len,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                        uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                        int saguaro, float eps, int32_t* cand, int32_t* hit, int32_t* cand_idx,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!cand || (saguaro != 0 && saguaro != 1)) return SPEC_EINVAL;
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, saguaro,
                         eps, cand, hit, cand_idx);
}

int spec_verify_early(const void* draft_logits, const void* target_logits, int dtype,
                      const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                      int B, int gamma, int V, float temperature, const int32_t* in_len,
                      int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                      uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                      int saguaro, float eps, void* workspace, size_t workspace_bytes, void* stream) {
  if (saguaro != 0 && saguaro != 1) return SPEC_EINVAL;
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream, saguaro,
                         eps, nullptr, nullptr, nullptr, 1);
}

int spec_verify_ex(const void* draft_logits, const void* target_logits, int dtype,
                   const int32_t* draft_tokens, const float* u_accept, const float* u_sample, int B,
                   int gamma, int V, float temperature, const int32_t* in_len, int32_t* out_tokens,
                   int32_t* out_accepted, int32_t* out_first_reject, uint64_t* out_accept_mask,
                   int32_t* out_len, const spec_diag* diag, const spec_options* opts,
                   void* workspace, size_t workspace_bytes, void* stream) {
  spec_options o{};
  if (opts) o = *opts;
  if (o.saguaro != 0 && o.saguaro != 1) return SPEC_EINVAL;
  if (o.early && o.cand) return SPEC_EINVAL;
  if (!(o.top_p >= 0.f && o.top_p <= 1.f)) return SPEC_EINVAL;   // NaN included
  const float top_p = o.top_p > 0.f ? o.top_p : 1.f;
  if (o.early && top_p < 1.f) return SPEC_EINVAL;
  if (!o.cand && (o.hit || o.cand_idx)) return SPEC_EINVAL;
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, workspace, workspace_bytes, stream,
                         o.saguaro, o.saguaro ? o.eps : 0.f, o.cand, o.hit, o.cand_idx, o.early ? 1 : 0,
                         o.temperature, top_p);
}

#if SV_CHECKS
// Present only in the checks build: lets a caller confirm which library it loaded.
int spec_checks_build(void) { return 1; }
#endif

#if SV_TIMELINE
// Measurement build only (not declared in spec_verify.h): copies n uint4
// words (two per block, see g_timeline) of the last single-kernel launch to
// host memory `dst`.  Synchronous.
int spec_timeline_copy(void* dst, size_t n) {
  if (!dst) return SPEC_EINVAL;
  n = std::min<size_t>(n, 2 * (size_t)sv::kTimelineBlocks);
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(sv::g_timeline), n * sizeof(uint4), 0,
                             hipMemcpyDeviceToHost) == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}
#endif

int spec_verify_noalloc(const void* draft_logits, const void* target_logits, int dtype,
                        const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                        int B, int gamma, int V, float temperature, const int32_t* in_len,
                        int32_t* out_tokens, int32_t* out_accepted, int32_t* out_first_reject,
                        uint64_t* out_accept_mask, int32_t* out_len, const spec_diag* diag,
                        void* stream) {
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (!sv::sizes_ok(B, gamma, V)) return SPEC_EINVAL;
  if (B == 0) return SPEC_OK;
  const size_t need = sv::layout(B, gamma, V).total;
  if (need > sv::kScratchBytes) return SPEC_ESCRATCH;
  void* ws = nullptr;
  if (sv::scratch_address(ws) != hipSuccess) return SPEC_ELAUNCH;
  // The workspace protocol wants it zero on entry; a completed call leaves it
  // so, but one whose wait gave up does not, so every call clears it first.
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const size_t n16 = (need + 15) / 16;
  const unsigned grid = (unsigned)std::min<size_t>((n16 + sv::kThreads * 4 - 1) / (sv::kThreads * 4), 2048);
  hipLaunchKernelGGL(sv::zero_kernel, dim3(grid), dim3(sv::kThreads), 0, st, static_cast<uint4*>(ws), n16);
  if (hipGetLastError() != hipSuccess) return SPEC_ELAUNCH;
  return sv::verify_impl(draft_logits, target_logits, dtype, draft_tokens, u_accept, u_sample, B,
                         gamma, V, temperature, in_len, out_tokens, out_accepted, out_first_reject,
                         out_accept_mask, out_len, diag, ws, sv::kScratchBytes, stream, 0, 0.f);
}

const char* spec_status_str(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument (size, temperature, eps or NULL pointer)";
    case SPEC_EDTYPE: return "unknown dtype (expected SPEC_F32 or SPEC_BF16)";
    case SPEC_EWORKSPACE: return "workspace missing or smaller than spec_workspace_bytes()";
    case SPEC_ELAUNCH: return "kernel launch failed";
    case SPEC_ESCRATCH: return "sizes need more workspace than spec_verify_noalloc's static scratch (16 MiB)";
    default: return "unknown status";
  }
}

}  // extern "C"
