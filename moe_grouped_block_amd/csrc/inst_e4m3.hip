// Instances of the fused kernel for one operand family (e4m3).
#include "grouped_gemm.h"

namespace moegg {

hipError_t launch_e4m3(int act, int out, const KernelArgs& a, hipStream_t s) {
  return launch_family<AB_E4M3>(act, out, a, s);
}

}  // namespace moegg
