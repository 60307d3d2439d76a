// Instantiations of the bf16 matrix-core GEMM for the forward products X W^T (both operands k-contiguous).
#include "gemm_mfma_kernel.h"

namespace gk {
void gemm_mfma_run_kk(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s) {
    run_cfg<true, true>(g, p, part, s);
}
}  // namespace gk
