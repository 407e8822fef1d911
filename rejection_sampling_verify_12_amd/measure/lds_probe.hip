// A measurement aid, built into the library beside the verification (and
// outside its kernel sources): LDS atomic adds in fixed lane-to-word
// patterns, the cost the top-p counting kernel's counter layout is designed
// around.  One 1024-thread work-group per CU, as the counting kernel runs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "spec_verify.h"

namespace {

constexpr int kProbeThreads = 1024;
constexpr int kProbeWords = 32768;   // 128 KB: 2048 words per wave

// Every wave adds 1 to words of its own 2048-word region, 8 adds per
// iteration, lane l to word: 0: l (64 words, 64 banks); 1: l / 8 (8 words,
// 8 lanes each); 2: 0 (one word); 3: 64 (l mod 32) (32 words on one bank).
__global__ __launch_bounds__(kProbeThreads) void lds_probe_kernel(int pattern, int iters, uint64_t* sink) {
  __shared__ uint32_t cnt[kProbeWords];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int i = t; i < kProbeWords; i += kProbeThreads) cnt[i] = 0u;
  __syncthreads();
  uint32_t w = 0u;
  if (pattern == 0) w = (uint32_t)lane;
  else if (pattern == 1) w = (uint32_t)lane >> 3;
  else if (pattern == 3) w = 64u * (uint32_t)(lane & 31);
  uint32_t* p = cnt + 2048 * wave + w;   // w < 2048
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  if (t == 0 && cnt[2048 * wave] == 0xFFFFFFFFu) *sink = 1u;   // never true: keeps the adds
}

}  // namespace

extern "C" int spec_lds_atomic_probe(int pattern, int iters, uint64_t* sink, void* stream) {
  if (pattern < 0 || pattern > 3 || iters < 1 || iters > (1 << 20) || !sink) return SPEC_EINVAL;
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
    return SPEC_ELAUNCH;
  (void)hipGetLastError();
  hipLaunchKernelGGL(lds_probe_kernel, dim3((unsigned)ncu), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     pattern, iters, sink);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}
