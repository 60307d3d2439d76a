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
        float a, da;
        act_and_grad_rt(g.act, acc + g.bias[n], a, da);
        ((TC*)g.C)[o] = from_f32<TC>(da);
        ((TC*)g.C2)[o] = from_f32<TC>(a);
    } else if constexpr (EPI == EPI_BIAS_RESID) {
        ((float*)g.C)[o] = g.resid[o] + (acc + g.bias[n]);
    } else if constexpr (EPI == EPI_ACT_GRAD) {
        ((TC*)g.C)[o] = from_f32<TC>(acc * to_f32(((const TC*)g.aux)[o]));
    } else {   // EPI_ACCUM
        ((float*)g.C)[o] += acc;
    }
}

// Eight consecutive outputs (m, n .. n+7) of one row, 16-byte aligned, all
// inside the matrix, in two parts so that a caller can issue the loads of
// several chunks before their stores: epi_load reads what the epilogue needs
// besides the accumulators (the residual, the activation derivative or the
// previous gradient), epi_store applies the operation and stores. bias holds
// the eight column biases (or zeros); yout (ACT_GRAD only) receives the fp32
// values before storage rounding.
struct EpiIn {
    float4 a, b;      // fp32 residual / previous gradient
    bf16x8 h;         // bf16 derivative of the activation
};

template <typename TC, int EPI>
GPT_DEV EpiIn epi_load(const Gemm& g, int m, int n) {
    const int64_t o = (int64_t)m * g.ldc + n;
    EpiIn in;
    if constexpr (EPI == EPI_BIAS_RESID) {
        const float* r = g.resid + o;
        in.a = reinterpret_cast<const float4*>(r)[0];
        in.b = reinterpret_cast<const float4*>(r)[1];
    } else if constexpr (EPI == EPI_ACCUM) {
        const float* c = (const float*)g.C + o;
        in.a = reinterpret_cast<const float4*>(c)[0];
        in.b = reinterpret_cast<const float4*>(c)[1];
    } else if constexpr (EPI == EPI_ACT_GRAD) {
        static_assert(sizeof(TC) == 2, "the matrix-core ACT_GRAD epilogue stores bf16");
        in.h = *reinterpret_cast<const bf16x8*>((const TC*)g.aux + o);
    }
    return in;
}

template <typename TC, int EPI, int ACT>
GPT_DEV void epi_store(const Gemm& g, int m, int n, const float (&acc)[8], const float (&bias)[8], const EpiIn& in,
                       float* yout = nullptr) {
    const int64_t o = (int64_t)m * g.ldc + n;
    auto put = [&](void* base, const float (&x)[8]) {
        if constexpr (sizeof(TC) == 2) {
            bf16x8 b;
#pragma unroll
            for (int e = 0; e < 8; ++e) b[e] = (bf16)x[e];
            *reinterpret_cast<bf16x8*>((bf16*)base + o) = b;
        } else {
            float* p = (float*)base + o;
            reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
            reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
        }
    };
    float y[8];
    if constexpr (EPI == EPI_STORE) {
        put(g.C, acc);
    } else if constexpr (EPI == EPI_BIAS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = acc[e] + bias[e];
        put(g.C, y);
    } else if constexpr (EPI == EPI_BIAS_ACT) {
        float h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) act_and_grad<ACT>(acc[e] + bias[e], h[e], y[e]);
        put(g.C, y);
        put(g.C2, h);
    } else if constexpr (EPI == EPI_BIAS_RESID || EPI == EPI_ACCUM) {
        const float rv[8] = {in.a.x, in.a.y, in.a.z, in.a.w, in.b.x, in.b.y, in.b.z, in.b.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = rv[e] + (EPI == EPI_BIAS_RESID ? acc[e] + bias[e] : acc[e]);
        put(g.C, y);
    } else {   // EPI_ACT_GRAD
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = acc[e] * (float)in.h[e];
        put(g.C, y);
        if (yout) {
#pragma unroll
            for (int e = 0; e < 8; ++e) yout[e] = y[e];
        }
    }
}

template <typename TC, int EPI, int ACT>
GPT_DEV void epilogue_chunk8(const Gemm& g, int m, int n, const float (&acc)[8], const float (&bias)[8],
                             float* yout = nullptr) {
    const EpiIn in = epi_load<TC, EPI>(g, m, n);
    epi_store<TC, EPI, ACT>(g, m, n, acc, bias, in, yout);
}

void gemm_simple(const Gemm& g, hipStream_t s);
bool gemm_mfma_ok(const Gemm& g);
GemmPlan gemm_mfma_plan(const Gemm& g, size_t nscratch);
void gemm_mfma_main(const Gemm& g, const GemmPlan& p, float* scratch, hipStream_t s);
void gemm_mfma_reduce(const Gemm& g, const GemmPlan& p, const float* scratch, hipStream_t s);

}  // namespace gk
