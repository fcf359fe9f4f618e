// Instantiations of the GEMM kernel family for FP8 E4M3 weights in 2 KB tiles with FP32
// block scales (the GEMMs of FP8 checkpoints, routed beside the W12 ones).
#include "w12_gemm_kernel.h"

namespace w12 {

hipError_t launch_gemm_f8_src(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  return launch_gemm_src<SRC_F8>(a, epi, p, s);
}

}  // namespace w12
