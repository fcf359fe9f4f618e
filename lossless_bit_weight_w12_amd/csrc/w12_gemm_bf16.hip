// Instantiations of the GEMM kernel family for plain BF16 weights (the baseline).
#include "w12_gemm_kernel.h"

namespace w12 {

hipError_t launch_gemm_bf16_src(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  return launch_gemm_src<SRC_BF16>(a, epi, p, s);
}

}  // namespace w12
