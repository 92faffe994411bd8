// Test support (not part of the FMHA library): fills the LDS of every CU with
// NaN bit patterns, so that a later kernel that reads LDS it never wrote turns
// its output non-finite instead of silently reusing stale values.
#include <hip/hip_runtime.h>

namespace {

constexpr int kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU
constexpr int kThreads = 1024;

__global__ __launch_bounds__(kThreads) void lds_poison_kernel() {
  extern __shared__ unsigned lds[];
  for (int i = threadIdx.x; i < kLdsBytes / 4; i += kThreads) lds[i] = 0x7fc07fc0u;
  __syncthreads();
}

}  // namespace

// Launches enough one-workgroup-per-CU waves (workgroups x 160 KB) to cover
// every CU twice. Returns 0 on success, the HIP error code otherwise.
extern "C" int lds_poison_launch(int workgroups, void* stream) {
  hipError_t e = hipFuncSetAttribute((const void*)lds_poison_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(lds_poison_kernel, dim3(workgroups), dim3(kThreads), kLdsBytes,
                     (hipStream_t)stream);
  return (int)hipGetLastError();
}
