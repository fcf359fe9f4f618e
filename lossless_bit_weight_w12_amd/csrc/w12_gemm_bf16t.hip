// Instantiations of the GEMM kernel family for BF16 weights in 4 KB tiles (the second
// baseline: the same streaming structure as W12 with 16 bits per weight).
#include "w12_gemm_kernel.h"

namespace w12 {

hipError_t launch_gemm_bf16t_src(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  return launch_gemm_src<SRC_BF16T>(a, epi, p, s);
}

}  // namespace w12
