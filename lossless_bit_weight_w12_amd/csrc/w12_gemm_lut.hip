// Instantiations of the GEMM kernel family for W12 weights with an arbitrary ascending
// codebook (16-entry byte lookup).
#include "w12_gemm_kernel.h"

namespace w12 {

hipError_t launch_gemm_lut(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  return launch_gemm_src<SRC_LUT>(a, epi, p, s);
}

}  // namespace w12
