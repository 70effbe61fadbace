// Kernel dispatch of libmoegg: routes a call to the instances of its operand
// family (inst_*.hip, one translation unit each), the amax fill kernel and
// the scale-layout conversion.
#include <hip/hip_runtime.h>

#include "moegg_internal.h"

namespace moegg {
namespace {

__global__ void fill_zero_kernel(float* ptr, int count) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < count) ptr[i] = 0.0f;
}

// One 32-bit scale word per thread: word w (128 K elements) of row r moves
// from r * words + w (row-major) to w * rows + r (K-block planes).  Threads
// run along the rows of one plane (blockIdx.y), so the writes are contiguous.
__global__ void sf_kplanes_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst, int64_t rows,
                                  int words) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int w = static_cast<int>(blockIdx.y);
  if (r < rows) dst[static_cast<int64_t>(w) * rows + r] = src[r * words + w];
}

}  // namespace

hipError_t launch_sf_kplanes(const uint8_t* src, uint8_t* dst, int64_t rows, int words, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int64_t bx = (rows + 255) / 256;
  if (bx > 0x7FFFFFFF || words <= 0 || words > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sf_kplanes_kernel, dim3(static_cast<unsigned>(bx), static_cast<unsigned>(words)), dim3(256), 0, s,
                     reinterpret_cast<const uint32_t*>(src), reinterpret_cast<uint32_t*>(dst), rows, words);
  return hipGetLastError();
}

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
