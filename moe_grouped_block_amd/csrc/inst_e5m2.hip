// Instances of the fused kernel for one operand family (e5m2).
#include "grouped_gemm.h"

namespace moegg {

hipError_t launch_e5m2(int act, int out, const KernelArgs& a, hipStream_t s) {
  return launch_family<AB_E5M2>(act, out, a, s);
}

}  // namespace moegg
