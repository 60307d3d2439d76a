// Muon for the hidden matrices of the blocks.
//
// The Modded-NanoGPT README's technique list names Muon and links its
// article (K. Jordan et al., "Muon: An optimizer for hidden layers in neural
// networks", 2024), which defines it: for a weight W [r, c] with gradient g
// and momentum buffer B,
//     B <- mu B + g,  u = g + mu B                        (Nesterov)
//     X0 = u' / (|u|_F + 1e-7), u' = u taken wide (transposed when r > c)
//     five times:  A = X X^T,  X <- a X + (b A + c A A) X
//     W <- W - lr sqrt(max(1, r / c)) X (oriented back)
// with (a, b, c) = (3.4445, -4.7750, 2.0315).
//
// The three products of an iteration run on the training step's GEMM (matrix
// cores for bf16 models): A = X X^T (both operands k-contiguous), A A (the
// second operand read row-major) and (a I + b A + c A A) X, where the a X term
// is folded into the left factor's diagonal so that one product and no extra
// pass over X finish the iteration. The elementwise steps are small kernels:
// momentum and direction with the transpose through LDS and per-tile sums of
// squares, the norm (summed in a fixed order), the normalisation, the
// polynomial in A, and the update (transposed back through LDS, bf16 shadow
// refreshed). Matrix X is stored bf16 for bf16 models (fp32 accumulation in
// every product) and fp32 otherwise.
#include "common.h"
#include "kernels.h"

namespace gk {

namespace {

constexpr int MT = 64;   // tile edge of the transposing kernels

}  // namespace

// buf <- mu buf + coef g and u = coef g + mu buf for W [r, c]; u is written
// [c, r] when tr (X = W^T), else [r, c]. part[tile] = sum of u^2 over the
// tile. Nothing is written when *nonfinite is set (the update is skipped).
__global__ __launch_bounds__(256) void muon_momentum_kernel(const float* __restrict__ g, float* __restrict__ buf,
                                                            float* __restrict__ u, float* __restrict__ part, int r,
                                                            int c, int tr, float mu, const float* __restrict__ coef_p,
                                                            const int32_t* __restrict__ nonfinite) {
    if (*nonfinite) return;
    __shared__ float tile[MT][MT + 1];
    __shared__ float red[4];
    const int r0 = blockIdx.y * MT, c0 = blockIdx.x * MT;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const float coef = *coef_p;
    float ss = 0.f;
#pragma unroll 4
    for (int i = ty; i < MT; i += 4) {
        const int row = r0 + i, col = c0 + tx;
        float v = 0.f;
        if (row < r && col < c) {
            const int64_t o = (int64_t)row * c + col;
            const float gv = coef * g[o];
            const float b = mu * buf[o] + gv;
            buf[o] = b;
            v = gv + mu * b;
            if (!tr) u[o] = v;
        }
        tile[i][tx] = v;
        ss += v * v;
    }
    if (tr) {
        __syncthreads();
        // u [c, r]: row c0 + i, columns r0 + tx (coalesced), from tile[tx][i]
#pragma unroll 4
        for (int i = ty; i < MT; i += 4) {
            const int row = c0 + i, col = r0 + tx;
            if (row < c && col < r) u[(int64_t)row * r + col] = tile[tx][i];
        }
    }
    ss = wave_sum(ss);
    if (tx == 0) red[ty] = ss;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// scale[0] = 1 / (sqrt(sum of part) + eps), summed by one workgroup in a fixed order
__global__ __launch_bounds__(256) void muon_norm_kernel(const float* __restrict__ part, int np, float eps,
                                                        float* __restrict__ scale) {
    __shared__ double red[4];
    double s = 0.0;
    for (int i = threadIdx.x; i < np; i += 256) s += (double)part[i];
    s = wave_sum_d(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) scale[0] = (float)(1.0 / (sqrt((red[0] + red[1]) + (red[2] + red[3])) + (double)eps));
}

// X_e = u_e * scale[e] for the entries e of a batch of mn-element matrices (storage TX)
template <typename TX>
__global__ __launch_bounds__(256) void muon_scale_kernel(const float* __restrict__ u, TX* __restrict__ X, int64_t mn,
                                                         int batch, const float* __restrict__ scale) {
    const int e = blockIdx.y;
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= mn) return;
    const float s = scale[e];
    const float* ue = u + e * mn;
    TX* xe = X + e * mn;
    if (i + 4 <= mn && mn % 4 == 0) {
        const float4 v = load4(ue + i);
        store4(xe + i, make_float4(v.x * s, v.y * s, v.z * s, v.w * s));
    } else {
        const int64_t end = i + 4 < mn ? i + 4 : mn;
        for (int64_t j = i; j < end; ++j) xe[j] = (TX)(ue[j] * s);
    }
}

// Bp = a I + b A + c AA over a batch of [m, m] matrices
template <typename TX>
__global__ __launch_bounds__(256) void muon_poly_kernel(const TX* __restrict__ A, const TX* __restrict__ AA,
                                                        TX* __restrict__ Bp, int m, int64_t total, float a, float b,
                                                        float c) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t k = i % ((int64_t)m * m);
    const int row = (int)(k / m), col = (int)(k - (int64_t)row * m);
    float v = b * (float)A[i] + c * (float)AA[i];
    if (row == col) v += a;
    Bp[i] = (TX)v;
}

// W [r, c] -= step * O with O = X^T (X [c, r]) when tr, else X [r, c]; the bf16
// shadow (wbf, nullable) gets the new values. Skipped when *nonfinite is set.
template <typename TX>
__global__ __launch_bounds__(256) void muon_apply_kernel(float* __restrict__ W, bf16* __restrict__ wbf,
                                                         const TX* __restrict__ X, int r, int c, int tr, float step,
                                                         const int32_t* __restrict__ nonfinite) {
    if (*nonfinite) return;
    __shared__ float tile[MT][MT + 1];
    const int r0 = blockIdx.y * MT, c0 = blockIdx.x * MT;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    if (tr) {
        // X rows c0 + i, columns r0 + tx (coalesced) into tile[i][tx]
#pragma unroll 4
        for (int i = ty; i < MT; i += 4) {
            const int row = c0 + i, col = r0 + tx;
            tile[i][tx] = (row < c && col < r) ? (float)X[(int64_t)row * r + col] : 0.f;
        }
        __syncthreads();
    }
#pragma unroll 4
    for (int i = ty; i < MT; i += 4) {
        const int row = r0 + i, col = c0 + tx;
        if (row < r && col < c) {
            const int64_t o = (int64_t)row * c + col;
            const float x = tr ? tile[tx][i] : (float)X[o];
            const float nw = W[o] - step * x;
            W[o] = nw;
            if (wbf) wbf[o] = (bf16)nw;
        }
    }
}

int64_t muon_part_floats(int r, int c) { return (int64_t)ceil_div(r, MT) * ceil_div(c, MT); }

void muon_direction(const float* g, float* buf, float* u, float* part, int r, int c, float mu, const float* coef,
                    const int32_t* nonfinite, float* scale, hipStream_t s) {
    const dim3 grid(ceil_div(c, MT), ceil_div(r, MT));
    muon_momentum_kernel<<<grid, 256, 0, s>>>(g, buf, u, part, r, c, r > c ? 1 : 0, mu, coef, nonfinite);
    muon_norm_kernel<<<1, 256, 0, s>>>(part, (int)(grid.x * grid.y), 1e-7f, scale);
}

// Five Newton-Schulz iterations on a batch of matrices X_e [m, n] (m <= n),
// X_e = u_e * scale[e] with u_e at u + e m n. X0 and X1 hold batch * m * n
// elements, A, AA, Bp batch * m * m (storage bf16 when bf); the products of
// all entries run as one batched launch each. Returns the buffer that holds
// the results (X1: an odd number of iterations).
void* muon_newton_schulz(bool bf, const float* u, const float* scale, int m, int n, int batch, void* X0, void* X1,
                         void* A, void* AA, void* Bp, float* splitk, size_t splitk_floats, hipStream_t s) {
    const int64_t mn = (int64_t)m * n, mm = (int64_t)m * m;
    const dim3 gs((unsigned)ceil_div(ceil_div(mn, (int64_t)4), (int64_t)256), (unsigned)batch);
    if (bf) muon_scale_kernel<bf16><<<gs, 256, 0, s>>>(u, (bf16*)X0, mn, batch, scale);
    else muon_scale_kernel<float><<<gs, 256, 0, s>>>(u, (float*)X0, mn, batch, scale);
    auto prod = [&](int M, int N, int K, const void* Ap, int64_t lda, int64_t sa, const void* Bq, int64_t ldb,
                    int64_t sb, bool b_kc, void* C, int64_t sc) {
        Gemm g{};
        g.M = M; g.N = N; g.K = K;
        g.A = Ap; g.lda = lda; g.a_kc = true;
        g.B = Bq; g.ldb = ldb; g.b_kc = b_kc;
        g.C = C; g.ldc = N; g.c_bf = bf;
        g.epi = EPI_STORE;
        g.in_bf = bf;
        g.batch = batch; g.sa = sa; g.sb = sb; g.sc = sc;
        gemm(g, splitk, splitk_floats, s);
    };
    void* X = X0;
    void* Y = X1;
    const unsigned nbm = (unsigned)ceil_div(batch * mm, (int64_t)256);
    for (int it = 0; it < 5; ++it) {
        prod(m, m, n, X, n, mn, X, n, mn, true, A, mm);       // A = X X^T
        prod(m, m, m, A, m, mm, A, m, mm, false, AA, mm);     // A A
        if (bf) muon_poly_kernel<bf16><<<nbm, 256, 0, s>>>((const bf16*)A, (const bf16*)AA, (bf16*)Bp, m, batch * mm,
                                                            3.4445f, -4.7750f, 2.0315f);
        else muon_poly_kernel<float><<<nbm, 256, 0, s>>>((const float*)A, (const float*)AA, (float*)Bp, m, batch * mm,
                                                          3.4445f, -4.7750f, 2.0315f);
        prod(m, n, m, Bp, m, mm, X, n, mn, false, Y, mn);     // (a I + b A + c A A) X
        std::swap(X, Y);
    }
    return X;
}

void muon_apply(bool bf, float* W, void* wbf, const void* X, int r, int c, float step, const int32_t* nonfinite,
                hipStream_t s) {
    const dim3 grid(ceil_div(c, MT), ceil_div(r, MT));
    const int tr = r > c ? 1 : 0;
    if (bf) muon_apply_kernel<bf16><<<grid, 256, 0, s>>>(W, (bf16*)wbf, (const bf16*)X, r, c, tr, step, nonfinite);
    else muon_apply_kernel<float><<<grid, 256, 0, s>>>(W, (bf16*)wbf, (const float*)X, r, c, tr, step, nonfinite);
}

}  // namespace gk
