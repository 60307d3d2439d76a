// Instantiations of the bf16 matrix-core GEMM for the weight gradients dY^T X (both operands row-contiguous).
#include "gemm_mfma_kernel.h"

namespace gk {
void gemm_mfma_run_cc(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s) {
    run_cfg<false, false>(g, p, part, s);
}
}  // namespace gk
