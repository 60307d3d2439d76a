// Instantiations of the bf16 matrix-core GEMM for the input gradients dY W (B row-contiguous).
#include "gemm_mfma_kernel.h"

namespace gk {
void gemm_mfma_run_kc(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s) {
    run_cfg<true, false>(g, p, part, s);
}
}  // namespace gk
