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

// Batch entry e = blockIdx.z: the matrix W_e [r, c] whose gradient and buffer
// start at g + e os and buf + e os. buf <- mu buf + coef g and u = coef g +
// mu buf; u_e (at u + e r c) is written [c, r] when tr (X = W^T), else [r, c];
// part[e ps + tile] = sum of u^2 over the tile. A 64 x 64 tile per workgroup,
// four consecutive columns per thread (VEC: 16-byte accesses, c % 4 == 0).
// Nothing is written when *nonfinite is set (the update is skipped).
template <bool VEC>
__global__ __launch_bounds__(256) void muon_momentum_kernel(const float* __restrict__ g, float* __restrict__ buf,
                                                            int64_t os, float* __restrict__ u, float* __restrict__ part,
                                                            int64_t ps, int r, int c, int tr, float mu,
                                                            const float* __restrict__ coef_p,
                                                            const int32_t* __restrict__ nonfinite) {
    if (*nonfinite) return;
    __shared__ float tile[MT][MT + 1];
    __shared__ float red[4];
    const int e = blockIdx.z;
    g += e * os;
    buf += e * os;
    u += (int64_t)e * r * c;
    const int r0 = blockIdx.y * MT, c0 = blockIdx.x * MT;
    const int cx = (threadIdx.x & 15) * 4, ty = threadIdx.x >> 4;
    const float coef = *coef_p;
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < MT / 16; ++p) {
        const int i = ty + 16 * p, row = r0 + i, col = c0 + cx;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (row < r) {
            const int64_t o = (int64_t)row * c + col;
            if (VEC && col < c) {
                const float4 gv = load4(g + o), bv = load4(buf + o);
                const float gg[4] = {coef * gv.x, coef * gv.y, coef * gv.z, coef * gv.w};
                const float bo[4] = {bv.x, bv.y, bv.z, bv.w};
                float nb[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    nb[k] = mu * bo[k] + gg[k];
                    v[k] = gg[k] + mu * nb[k];
                }
                store4(buf + o, make_float4(nb[0], nb[1], nb[2], nb[3]));
                if (!tr) store4(u + o, make_float4(v[0], v[1], v[2], v[3]));
            } else if (!VEC) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (col + k < c) {
                        const float gk_ = coef * g[o + k];
                        const float nb = mu * buf[o + k] + gk_;
                        buf[o + k] = nb;
                        v[k] = gk_ + mu * nb;
                        if (!tr) u[o + k] = v[k];
                    }
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            tile[i][cx + k] = v[k];
            ss += v[k] * v[k];
        }
    }
    if (tr) {
        __syncthreads();
        // u [c, r]: row c0 + i, columns r0 + cx .. + 3, from tile[cx + k][i]
#pragma unroll
        for (int p = 0; p < MT / 16; ++p) {
            const int i = ty + 16 * p, row = c0 + i, col = r0 + cx;
            if (row < c) {
                const int64_t o = (int64_t)row * r + col;
                if (VEC && (r & 3) == 0 && col < r) {
                    store4(u + o, make_float4(tile[cx][i], tile[cx + 1][i], tile[cx + 2][i], tile[cx + 3][i]));
                } else {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (col + k < r) u[o + k] = tile[cx + k][i];
                }
            }
        }
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0)
        part[e * ps + blockIdx.y * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// scale[e] = 1 / (sqrt(sum of part[e ps .. e ps + np)) + eps), one workgroup per
// entry, summed in a fixed order
__global__ __launch_bounds__(256) void muon_norm_kernel(const float* __restrict__ part, int np, int64_t ps, float eps,
                                                        float* __restrict__ scale) {
    __shared__ double red[4];
    const int e = blockIdx.x;
    double s = 0.0;
    for (int i = threadIdx.x; i < np; i += 256) s += (double)part[e * ps + i];
    s = wave_sum_d(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) scale[e] = (float)(1.0 / (sqrt((red[0] + red[1]) + (red[2] + red[3])) + (double)eps));
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

// Bp = a I + b A + c AA over a batch of [m, m] matrices, four elements per
// thread (16-byte fp32 or 8-byte bf16 accesses when m % 4 == 0)
template <typename TX>
__global__ __launch_bounds__(256) void muon_poly_kernel(const TX* __restrict__ A, const TX* __restrict__ AA,
                                                        TX* __restrict__ Bp, int m, int64_t total, float a, float b,
                                                        float c) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= total) return;
    const int64_t mm = (int64_t)m * m;
    if ((m & 3) == 0) {
        const float4 x = load4(A + i), y = load4(AA + i);
        float v[4] = {b * x.x + c * y.x, b * x.y + c * y.y, b * x.z + c * y.z, b * x.w + c * y.w};
        const int64_t k = i % mm;
        const int row = (int)(k / m), col = (int)(k - (int64_t)row * m);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (row == col + q) v[q] += a;
        store4(Bp + i, make_float4(v[0], v[1], v[2], v[3]));
    } else {
        const int64_t end = i + 4 < total ? i + 4 : total;
        for (int64_t j = i; j < end; ++j) {
            const int64_t k = j % mm;
            const int row = (int)(k / m), col = (int)(k - (int64_t)row * m);
            float v = b * (float)A[j] + c * (float)AA[j];
            if (row == col) v += a;
            Bp[j] = (TX)v;
        }
    }
}

// Batch entry e = blockIdx.z: W_e [r, c] (at W + e os, bf16 shadow at wbf + e
// os, nullable) -= step * O with O = X_e^T (X_e [c, r] at X + e r c) when tr,
// else X_e [r, c]. Four consecutive columns per thread (VEC: 16-byte fp32
// accesses, c % 4 == 0 and r % 4 == 0). Skipped when *nonfinite is set.
template <typename TX, bool VEC>
__global__ __launch_bounds__(256) void muon_apply_kernel(float* __restrict__ W, bf16* __restrict__ wbf, int64_t os,
                                                         const TX* __restrict__ X, int r, int c, int tr, float step,
                                                         const int32_t* __restrict__ nonfinite) {
    if (*nonfinite) return;
    __shared__ float tile[MT][MT + 1];
    const int e = blockIdx.z;
    W += e * os;
    if (wbf) wbf += e * os;
    X += (int64_t)e * r * c;
    const int r0 = blockIdx.y * MT, c0 = blockIdx.x * MT;
    const int cx = (threadIdx.x & 15) * 4, ty = threadIdx.x >> 4;
    if (tr) {
        // X rows c0 + i, columns r0 + cx .. + 3 (coalesced) into tile[i][cx + k]
#pragma unroll
        for (int p = 0; p < MT / 16; ++p) {
            const int i = ty + 16 * p, row = c0 + i, col = r0 + cx;
            float x[4] = {0.f, 0.f, 0.f, 0.f};
            if (row < c) {
                const int64_t o = (int64_t)row * r + col;
                if (VEC && col < r) {
                    const float4 v = load4(X + o);
                    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
                } else if (!VEC) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        if (col + k < r) x[k] = (float)X[o + k];
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) tile[i][cx + k] = x[k];
        }
        __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < MT / 16; ++p) {
        const int i = ty + 16 * p, row = r0 + i, col = c0 + cx;
        if (row >= r) continue;
        const int64_t o = (int64_t)row * c + col;
        if (VEC) {
            if (col >= c) continue;
            float x[4];
            if (tr) {
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] = tile[cx + k][i];
            } else {
                const float4 v = load4(X + o);
                x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
            }
            const float4 w0 = load4(W + o);
            const float4 nw = make_float4(w0.x - step * x[0], w0.y - step * x[1], w0.z - step * x[2],
                                          w0.w - step * x[3]);
            store4(W + o, nw);
            if (wbf) store4(wbf + o, nw);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (col + k < c) {
                    const float x = tr ? tile[cx + k][i] : (float)X[o + k];
                    const float nw = W[o + k] - step * x;
                    W[o + k] = nw;
                    if (wbf) wbf[o + k] = (bf16)nw;
                }
        }
    }
}

int64_t muon_part_floats(int r, int c) { return (int64_t)ceil_div(r, MT) * ceil_div(c, MT); }

void muon_direction(const float* g, float* buf, int64_t os, int batch, float* u, float* part, int64_t ps, int r, int c,
                    float mu, const float* coef, const int32_t* nonfinite, float* scale, hipStream_t s) {
    const dim3 grid(ceil_div(c, MT), ceil_div(r, MT), batch);
    const int tr = r > c ? 1 : 0;
    const bool vec = c % 4 == 0 && r % 4 == 0 && os % 4 == 0;
    if (vec) muon_momentum_kernel<true><<<grid, 256, 0, s>>>(g, buf, os, u, part, ps, r, c, tr, mu, coef, nonfinite);
    else muon_momentum_kernel<false><<<grid, 256, 0, s>>>(g, buf, os, u, part, ps, r, c, tr, mu, coef, nonfinite);
    muon_norm_kernel<<<batch, 256, 0, s>>>(part, (int)(grid.x * grid.y), ps, 1e-7f, scale);
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

void muon_apply(bool bf, float* W, void* wbf, int64_t os, int batch, const void* X, int r, int c, float step,
                const int32_t* nonfinite, hipStream_t s) {
    const dim3 grid(ceil_div(c, MT), ceil_div(r, MT), batch);
    const int tr = r > c ? 1 : 0;
    const bool vec = c % 4 == 0 && r % 4 == 0 && os % 4 == 0;
    if (bf && vec)
        muon_apply_kernel<bf16, true><<<grid, 256, 0, s>>>(W, (bf16*)wbf, os, (const bf16*)X, r, c, tr, step, nonfinite);
    else if (bf)
        muon_apply_kernel<bf16, false><<<grid, 256, 0, s>>>(W, (bf16*)wbf, os, (const bf16*)X, r, c, tr, step, nonfinite);
    else if (vec)
        muon_apply_kernel<float, true><<<grid, 256, 0, s>>>(W, (bf16*)wbf, os, (const float*)X, r, c, tr, step, nonfinite);
    else
        muon_apply_kernel<float, false><<<grid, 256, 0, s>>>(W, (bf16*)wbf, os, (const float*)X, r, c, tr, step, nonfinite);
}

}  // namespace gk
