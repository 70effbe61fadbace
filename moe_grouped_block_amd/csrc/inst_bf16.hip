// Instances of the fused kernel for one operand family (bf16).
#include "grouped_gemm.h"

namespace moegg {

hipError_t launch_bf16(int act, int out, const KernelArgs& a, hipStream_t s) {
  return launch_family<AB_BF16>(act, out, a, s);
}

}  // namespace moegg
