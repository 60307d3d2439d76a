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

// The 16 values of one 32x32 accumulator fragment column: rows
// rb + 8*(e/4) + e%4 of column col, all inside the matrix. Every load the
// epilogue needs is issued before the first store.
template <typename TC, int EPI>
GPT_DEV void epilogue_frag(const Gemm& g, int rb, int col, const f32x16& acc, float bias) {
    const int64_t base = (int64_t)rb * g.ldc + col;
    auto off = [&](int e) { return base + (int64_t)(8 * (e >> 2) + (e & 3)) * g.ldc; };
    if constexpr (EPI == EPI_STORE) {
#pragma unroll
        for (int e = 0; e < 16; ++e) ((TC*)g.C)[off(e)] = from_f32<TC>(acc[e]);
    } else if constexpr (EPI == EPI_BIAS) {
#pragma unroll
        for (int e = 0; e < 16; ++e) ((TC*)g.C)[off(e)] = from_f32<TC>(acc[e] + bias);
    } else if constexpr (EPI == EPI_BIAS_ACT) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float pre = acc[e] + bias;
            ((TC*)g.C)[off(e)] = from_f32<TC>(pre);
            ((TC*)g.C2)[off(e)] = from_f32<TC>(g.act == ACT_RELU2 ? relu2_f(pre) : gelu_tanh_f(pre));
        }
    } else if constexpr (EPI == EPI_BIAS_RESID) {
        float r[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) r[e] = g.resid[off(e)];
#pragma unroll
        for (int e = 0; e < 16; ++e) ((float*)g.C)[off(e)] = r[e] + (acc[e] + bias);
    } else if constexpr (EPI == EPI_ACT_GRAD) {
        float x[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = to_f32(((const TC*)g.aux)[off(e)]);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            ((TC*)g.C)[off(e)] =
                from_f32<TC>(acc[e] * (g.act == ACT_RELU2 ? relu2_grad_f(x[e]) : gelu_tanh_grad_f(x[e])));
    } else {   // EPI_ACCUM
        float c[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) c[e] = ((float*)g.C)[off(e)];
#pragma unroll
        for (int e = 0; e < 16; ++e) ((float*)g.C)[off(e)] = c[e] + acc[e];
    }
}

void gemm_simple(const Gemm& g, hipStream_t s);
bool gemm_mfma_ok(const Gemm& g);
void gemm_mfma(const Gemm& g, float* scratch, size_t nscratch, hipStream_t s);

}  // namespace gk
