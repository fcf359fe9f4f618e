// Instantiations of the GEMM kernel family for W12 weights whose codebook is a run of
// 16 consecutive exponent fields (exponent = C[0] + code).
#include "w12_gemm_kernel.h"

namespace w12 {

hipError_t launch_gemm_run(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  return launch_gemm_src<SRC_RUN>(a, epi, p, s);
}

}  // namespace w12
