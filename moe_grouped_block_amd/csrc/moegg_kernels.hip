// Kernel dispatch of libmoegg: routes a call to the instances of its operand
// family (inst_*.hip, one translation unit each) and the amax fill kernel.
#include <hip/hip_runtime.h>

#include "moegg_internal.h"

namespace moegg {
namespace {

__global__ void fill_zero_kernel(float* ptr, int count) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < count) ptr[i] = 0.0f;
}

}  // namespace

hipError_t launch_grouped_gemm(int ab, int act, int out, const KernelArgs& a, hipStream_t s) {
  if (a.grid <= 0) return hipErrorInvalidValue;
  switch (ab) {
    case AB_E4M3: return launch_e4m3(act, out, a, s);
    case AB_E2M1: return launch_e2m1(act, out, a, s);
    case AB_BF16: return launch_bf16(act, out, a, s);
    case AB_E5M2: return launch_e5m2(act, out, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill_zero(float* ptr, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((count + 255) / 256), dim3(256), 0, s, ptr, count);
  return hipGetLastError();
}

}  // namespace moegg
