// A timed stand-in for a model forward pass, for pipeline experiments around
// the verification ("Speculative Speculative Decoding (Saguaro)", section 4.1:
// the draft model runs on its own stream (and device) while the target
// verifies; SSD summary, AMD MI300X part: draft and target on separate HIP
// streams synchronised by events).  No model weights exist here, so a "model"
// is a kernel that keeps one work-group busy for a set wall time: it occupies
// its stream for that long without taking the compute units the verification
// uses, as a model on a separate device would.
#include "spec_verify.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

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
