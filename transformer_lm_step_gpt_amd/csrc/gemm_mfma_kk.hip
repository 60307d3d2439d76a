// Instantiations of the bf16 matrix-core GEMM for the forward products X W^T (both operands k-contiguous).
#include "gemm_mfma_kernel.h"

namespace gk {
void gemm_mfma_run_kk(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s) {
    run_cfg<true, true>(g, p, part, s);
}

void gemm_mfma_run_f8(const Gemm& g, hipStream_t s) {
    const dim3 grid(ceil_div(g.N, 256) * ceil_div(g.M, 256), 1, 1);
    launch<256, 256, 64, 2, 1, PIPE_F8, 2, 4, true, true, EPI_STORE, 1, 0, false>(g, grid, g.K, nullptr, s);
}
}  // namespace gk
