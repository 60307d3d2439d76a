// Epilogue shared by the GEMM kernels: applies the fused operation to one
// accumulated fp32 value at (m, n).
#pragma once
#include "common.h"
#include "kernels.h"

namespace gk {

template <typename TC, int EPI>
GPT_DEV void epilogue_store(const Gemm& g, int m, int n, float acc) {
    const int64_t o = (int64_t)m * g.ldc + n;
    if constexpr (EPI == EPI_STORE) {
        ((TC*)g.C)[o] = from_f32<TC>(acc);
    } else if constexpr (EPI == EPI_BIAS) {
        ((TC*)g.C)[o] = from_f32<TC>(acc + g.bias[n]);
    } else if constexpr (EPI == EPI_BIAS_ACT) {
        float pre = acc + g.bias[n];
        ((TC*)g.C)[o] = from_f32<TC>(pre);
        ((TC*)g.C2)[o] = from_f32<TC>(g.act == ACT_RELU2 ? relu2_f(pre) : gelu_tanh_f(pre));
    } else if constexpr (EPI == EPI_BIAS_RESID) {
        ((float*)g.C)[o] = g.resid[o] + (acc + g.bias[n]);
    } else if constexpr (EPI == EPI_ACT_GRAD) {
        float pre = to_f32(((const TC*)g.aux)[o]);
        ((TC*)g.C)[o] = from_f32<TC>(acc * (g.act == ACT_RELU2 ? relu2_grad_f(pre) : gelu_tanh_grad_f(pre)));
    } else {   // EPI_ACCUM
        ((float*)g.C)[o] += acc;
    }
}

void gemm_simple(const Gemm& g, hipStream_t s);
bool gemm_mfma_ok(const Gemm& g);
void gemm_mfma(const Gemm& g, float* scratch, size_t nscratch, hipStream_t s);

}  // namespace gk
