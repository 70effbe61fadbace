// Instances of the fused kernel for one operand family (e2m1).
#include "grouped_gemm.h"

namespace moegg {

hipError_t launch_e2m1(int act, int out, const KernelArgs& a, hipStream_t s) {
  return launch_family<AB_E2M1>(act, out, a, s);
}

}  // namespace moegg
