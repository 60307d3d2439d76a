// General matrix products of the GPT-2 training step with fused epilogues.
//
// C[M, N] = epilogue(sum_k A(m, k) B(k, n)); A and B are read in either
// orientation so that the forward products (X W^T), the input gradients
// (dY W) and the weight gradients (dY^T X) all use the same kernels without
// transposed copies. Epilogues fuse the bias, the MLP activation (GELU tanh
// approximation or ReLU^2, "Раздел 1 / Архитектура" of the lecture notes;
// Modded-NanoGPT README technique list), the residual add, the activation
// derivative and gradient accumulation.
//
// This file holds the portable LDS-tiled FMA kernel (fp32 path and any shape);
// the bf16 matrix-core kernel is in gemm_mfma.hip.
#include "common.h"
#include "kernels.h"

#include <cstdio>
#include "gemm_common.h"

namespace gk {

template <typename TI, typename TC, int EPI>
__global__ __launch_bounds__(256) void gemm_simple_kernel(Gemm g) {
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const TI* A = (const TI*)g.A;
    const TI* B = (const TI*)g.B;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < g.K; k0 += BK) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            int idx = tid + 256 * e;
            int mm, kk;
            if (g.a_kc) { mm = idx >> 4; kk = idx & 15; } else { kk = idx >> 6; mm = idx & 63; }
            int gm = m0 + mm, gk = k0 + kk;
            float v = 0.f;
            if (gm < g.M && gk < g.K) v = to_f32(g.a_kc ? A[(int64_t)gm * g.lda + gk] : A[(int64_t)gk * g.lda + gm]);
            As[kk][mm] = v;
            int nn;
            if (g.b_kc) { nn = idx >> 4; kk = idx & 15; } else { kk = idx >> 6; nn = idx & 63; }
            int gn = n0 + nn;
            gk = k0 + kk;
            v = 0.f;
            if (gn < g.N && gk < g.K) v = to_f32(g.b_kc ? B[(int64_t)gn * g.ldb + gk] : B[(int64_t)gk * g.ldb + gn]);
            Bs[kk][nn] = v;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int m = m0 + ty + 16 * i;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int n = n0 + tx + 16 * j;
            if (n >= g.N) continue;
            epilogue_store<TC, EPI>(g, m, n, acc[i][j]);
        }
    }
}

template <typename TI, typename TC>
static void launch_simple_tc(const Gemm& g, hipStream_t s) {
    dim3 grid(ceil_div(g.N, 64), ceil_div(g.M, 64));
    switch (g.epi) {
        case EPI_STORE: gemm_simple_kernel<TI, TC, EPI_STORE><<<grid, 256, 0, s>>>(g); break;
        case EPI_BIAS: gemm_simple_kernel<TI, TC, EPI_BIAS><<<grid, 256, 0, s>>>(g); break;
        case EPI_BIAS_ACT: gemm_simple_kernel<TI, TC, EPI_BIAS_ACT><<<grid, 256, 0, s>>>(g); break;
        case EPI_BIAS_RESID: gemm_simple_kernel<TI, float, EPI_BIAS_RESID><<<grid, 256, 0, s>>>(g); break;
        case EPI_ACT_GRAD: gemm_simple_kernel<TI, TC, EPI_ACT_GRAD><<<grid, 256, 0, s>>>(g); break;
        case EPI_ACCUM: gemm_simple_kernel<TI, float, EPI_ACCUM><<<grid, 256, 0, s>>>(g); break;
    }
}

void gemm_simple(const Gemm& g, hipStream_t s) {
    if (g.in_bf) {
        if (g.c_bf) launch_simple_tc<bf16, bf16>(g, s);
        else launch_simple_tc<bf16, float>(g, s);
    } else {
        if (g.c_bf) launch_simple_tc<float, bf16>(g, s);
        else launch_simple_tc<float, float>(g, s);
    }
}

}  // namespace gk

namespace gk {
GemmPlan gemm_plan(const Gemm& g, size_t splitk_floats) {
    if (gemm_mfma_ok(g)) return gemm_mfma_plan(g, splitk_floats);
    GemmPlan p;
    snprintf(p.name, sizeof(p.name), "gemm_simple_kernel");
    return p;
}
void gemm_main(const Gemm& g, const GemmPlan& p, float* splitk_scratch, hipStream_t s) {
    if (p.cfg >= 0) gemm_mfma_main(g, p, splitk_scratch, s);
    else gemm_simple(g, s);
}
void gemm_finish(const Gemm& g, const GemmPlan& p, const float* splitk_scratch, hipStream_t s) {
    if (p.cfg >= 0) gemm_mfma_reduce(g, p, splitk_scratch, s);
}
void gemm(const Gemm& g, float* splitk_scratch, size_t splitk_floats, hipStream_t s) {
    if (g.batch > 1 && !gemm_mfma_ok(g)) {
        // the portable kernel takes one entry per launch
        Gemm e = g;
        e.batch = 1;
        const int64_t ea = g.in_bf ? 2 : 4, ec = g.c_bf ? 2 : 4;
        for (int b = 0; b < g.batch; ++b) {
            e.A = (const char*)g.A + b * g.sa * ea;
            e.B = (const char*)g.B + b * g.sb * ea;
            e.C = (char*)g.C + b * g.sc * ec;
            gemm_simple(e, s);
        }
        return;
    }
    const GemmPlan p = gemm_plan(g, g.batch > 1 ? 0 : splitk_floats);
    gemm_main(g, p, splitk_scratch, s);
    gemm_finish(g, p, splitk_scratch, s);
}
}  // namespace gk
