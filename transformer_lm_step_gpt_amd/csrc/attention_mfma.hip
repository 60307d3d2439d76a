// Matrix-core flash attention for gfx950, bf16 storage, head dims 64 and 128.
//
// Same mathematics as attention.hip (causal, optional window, online softmax,
// recompute in the backward pass; "El Mecanismo de Atención" of the speedrun
// baseline page and the FlashAttention / online-softmax paragraph of the
// lecture notes' "Раздел 2. Сделаем быстро"), mapped onto
// v_mfma_f32_32x32x16_bf16:
//
//   forward   S^T = K Q^T         each lane owns one query column, so the
//             O^T += V^T P^T      running max and sum need one cross-lane
//                                 shuffle, and P stays in registers as the
//                                 B operand of the second product;
//   dK, dV    S = Q K^T, dP = dO V^T (each lane owns one key column),
//             dV^T += dO^T P, dK^T += Q^T dS  (one workgroup per 128 keys);
//   dQ        S^T = K Q^T, dP^T = V dO^T (each lane owns one query),
//             dQ^T += K^T dS^T  (one workgroup per 128 queries).
//
// Accumulator fragments hold rows 8*(e/4) + 4*(lane/32) + e%4 of a 32-row
// block. When such a fragment is reused as the 16-deep k operand of the next
// product, k slot 8*(lane/32) + e' stands for row 8*(e'/4) + 4*(lane/32) +
// e'%4; the other operand is read from LDS with the same slot-to-row mapping
// (two 8-byte reads of 4 consecutive rows), so the product is unchanged.
//
// All outputs are written by exactly one workgroup: no atomics.
#include "common.h"
#include "kernels.h"

namespace gk {

namespace {

constexpr float M_LOG2E_F = 1.4426950408889634f;
constexpr float M_LN2_F = 0.6931471805599453f;
constexpr int ATT_BQ = 128;    // queries (fwd, dQ) or keys (dK dV) per workgroup: 4 waves x 32
constexpr int ATT_BT = 64;     // rows of the streamed tile

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

GPT_DEV int aswz(int row, int chunk, int nch) { return chunk ^ ((row >> 3) & (nch - 1)); }

GPT_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

GPT_DEV f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.f;
    return z;
}

// rows [r0, r0+ROWS) of a [T, HD] head slice into a row-major LDS tile
// (HD + 8 stride, 16-byte chunks swizzled by row / 8); rows >= T are zero
template <int HD, int ROWS>
GPT_DEV void stage_rows_major(bf16* dst, const bf16* src, int64_t ld, int r0, int T) {
    constexpr int CH = HD / 8, S = HD + 8, N = ROWS * CH;
    for (int c = threadIdx.x; c < N; c += 256) {
        int r = c / CH, ch = c % CH, gr = r0 + r;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (gr < T) v = *reinterpret_cast<const u32x4*>(src + (int64_t)gr * ld + ch * 8);
        *reinterpret_cast<u32x4*>(dst + r * S + aswz(r, ch, CH) * 8) = v;
    }
}

// the same rows transposed: dst[d][r] (stride ROWS + 4), via (r, r+1) pairs
template <int HD, int ROWS>
GPT_DEV void stage_cols_major(bf16* dst, const bf16* src, int64_t ld, int r0, int T) {
    constexpr int G = HD / 8, N = G * (ROWS / 2), S = ROWS + 4;
    for (int u = threadIdx.x; u < N; u += 256) {
        int g = u % G, r = 2 * (u / G), gr = r0 + r;
        u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
        if (gr < T) v0 = *reinterpret_cast<const u32x4*>(src + (int64_t)gr * ld + g * 8);
        if (gr + 1 < T) v1 = *reinterpret_cast<const u32x4*>(src + (int64_t)(gr + 1) * ld + g * 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t lo = (v0[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
            uint32_t hi = (v1[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
            *reinterpret_cast<uint32_t*>(dst + (g * 8 + i) * S + r) = lo | (hi << 16);
        }
    }
}

// 16-deep k operand from a row-major tile: row `row`, k = 16*ds + 8*(lane/32) + e
template <int HD>
GPT_DEV bf16x8 frag_rows(const bf16* t, int row, int ds, int hh) {
    constexpr int CH = HD / 8, S = HD + 8;
    return *reinterpret_cast<const bf16x8*>(t + row * S + aswz(row, 2 * ds + hh, CH) * 8);
}

// 16-deep k operand over permuted rows of a transposed tile: element d = `col`,
// rows 16*ks + 4*hh + {0..3} and 16*ks + 8 + 4*hh + {0..3}
template <int ROWS>
GPT_DEV bf16x8 frag_cols(const bf16* t, int col, int ks, int hh) {
    constexpr int S = ROWS + 4;
    const bf16* p = t + col * S + 16 * ks + 4 * hh;
    u32x2 lo = *reinterpret_cast<const u32x2*>(p);
    u32x2 hi = *reinterpret_cast<const u32x2*>(p + 8);
    u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, v);
}

GPT_DEV bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

GPT_DEV bool visible(int q, int key, int T, int W) {
    return key <= q && key < T && q < T && (W <= 0 || q - key < W);
}

}  // namespace

// ============================================================== forward

template <int HD>
__global__ __launch_bounds__(256) void attn_fwd_mfma_kernel(Attn a) {
    constexpr int NDS = HD / 16, NDF = HD / 32, SK = HD + 8;
    __shared__ __attribute__((aligned(16))) bf16 Ks[ATT_BT * SK];
    __shared__ __attribute__((aligned(16))) bf16 Vt[HD * (ATT_BT + 4)];
    const int qt = gridDim.x - 1 - blockIdx.x;   // heaviest query tiles first
    const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
    const int T = a.T, W = a.window;
    const int q0 = qt * ATT_BQ;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 31, hh = lane >> 5;
    const int qw = q0 + w * 32, myq = qw + lr;
    const bf16* Q = (const bf16*)a.q + (int64_t)b * T * a.ldq + h * HD;
    const bf16* K = (const bf16*)a.k + (int64_t)b * T * a.ldk + h * HD;
    const bf16* V = (const bf16*)a.v + (int64_t)b * T * a.ldv + h * HD;

    bf16x8 qf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        bf16x8 z = {};
        qf[ds] = myq < T ? load8(Q + (int64_t)myq * a.ldq + 16 * ds + 8 * hh) : z;
    }
    f32x16 oacc[NDF];
#pragma unroll
    for (int df = 0; df < NDF; ++df) oacc[df] = zero16();
    float mrow = -INFINITY, lsum = 0.f;
    const float c = M_LOG2E_F / sqrtf((float)HD);
    const int kend = min(T, q0 + ATT_BQ);
    int kbeg = W > 0 ? max(0, q0 - W + 1) : 0;
    kbeg = (kbeg / ATT_BT) * ATT_BT;
    for (int kt = kbeg; kt < kend; kt += ATT_BT) {
        __syncthreads();
        stage_rows_major<HD, ATT_BT>(Ks, K, a.ldk, kt, T);
        stage_cols_major<HD, ATT_BT>(Vt, V, a.ldv, kt, T);
        __syncthreads();
        if (kt > qw + 31) continue;                               // the whole tile is in this wave's future
        if (W > 0 && kt + ATT_BT - 1 <= qw - W) continue;          // the whole tile left every window
        f32x16 s[2];
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
            s[kf] = zero16();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s[kf] = mfma(frag_rows<HD>(Ks, kf * 32 + lr, ds, hh), qf[ds], s[kf]);
        }
        const bool need_mask = (kt + ATT_BT - 1 > qw) || (kt + ATT_BT > T) || (W > 0 && qw + 31 - kt >= W);
        float tmax = -INFINITY;
#pragma unroll
        for (int kf = 0; kf < 2; ++kf)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (need_mask) {
                    int key = kt + kf * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                    if (!visible(myq, key, T, W)) s[kf][e] = -INFINITY;
                }
                tmax = fmaxf(tmax, s[kf][e]);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mnew = fmaxf(mrow, tmax);
        const float mc = mnew == -INFINITY ? 0.f : mnew * c;
        const float corr = exp2f(mrow * c - mc);
        mrow = mnew;
        lsum *= corr;
#pragma unroll
        for (int df = 0; df < NDF; ++df)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[df][e] *= corr;
        bf16x8 pk[4];
#pragma unroll
        for (int kf = 0; kf < 2; ++kf)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float p = exp2f(fmaf(s[kf][e], c, -mc));
                lsum += p;
                pk[2 * kf + (e >> 3)][e & 7] = (bf16)p;
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int df = 0; df < NDF; ++df)
                oacc[df] = mfma(frag_cols<ATT_BT>(Vt, df * 32 + lr, ks, hh), pk[ks], oacc[df]);
    }
    const float l = lsum + __shfl_xor(lsum, 32, 64);
    if (myq < T) {
        const float inv = 1.0f / l;
        bf16* O = (bf16*)a.o + ((int64_t)b * T + myq) * a.ldo + h * HD;
#pragma unroll
        for (int df = 0; df < NDF; ++df)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = (bf16)(oacc[df][4 * g4 + i] * inv);
                *reinterpret_cast<bf16x4*>(O + df * 32 + 8 * g4 + 4 * hh) = v;
            }
        if (hh == 0) a.lse[(int64_t)bh * T + myq] = (mrow * c + log2f(l)) * M_LN2_F;
    }
}

// ============================================================== backward: dK, dV

template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_mfma_kernel(Attn a) {
    constexpr int NDS = HD / 16, NDF = HD / 32, SK = HD + 8, ST = ATT_BT + 4;
    __shared__ __attribute__((aligned(16))) bf16 Qs[ATT_BT * SK];
    __shared__ __attribute__((aligned(16))) bf16 Qt[HD * ST];
    __shared__ __attribute__((aligned(16))) bf16 Gs[ATT_BT * SK];   // dO rows
    __shared__ __attribute__((aligned(16))) bf16 Gt[HD * ST];       // dO transposed
    __shared__ float Ls[ATT_BT], Ds[ATT_BT];
    const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
    const int T = a.T, W = a.window;
    const int k0 = blockIdx.x * ATT_BQ;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 31, hh = lane >> 5;
    const int kw = k0 + w * 32, mykey = kw + lr;
    const bf16* Q = (const bf16*)a.q + (int64_t)b * T * a.ldq + h * HD;
    const bf16* K = (const bf16*)a.k + (int64_t)b * T * a.ldk + h * HD;
    const bf16* V = (const bf16*)a.v + (int64_t)b * T * a.ldv + h * HD;
    const bf16* G = (const bf16*)a.dO + (int64_t)b * T * a.lddo + h * HD;
    const float* LSE = a.lse + (int64_t)bh * T;
    const float* DD = a.D + (int64_t)bh * T;

    bf16x8 kf[NDS], vf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        bf16x8 z = {};
        kf[ds] = mykey < T ? load8(K + (int64_t)mykey * a.ldk + 16 * ds + 8 * hh) : z;
        vf[ds] = mykey < T ? load8(V + (int64_t)mykey * a.ldv + 16 * ds + 8 * hh) : z;
    }
    f32x16 dk[NDF], dv[NDF];
#pragma unroll
    for (int df = 0; df < NDF; ++df) { dk[df] = zero16(); dv[df] = zero16(); }
    const float c = M_LOG2E_F / sqrtf((float)HD);
    const int qbeg = (k0 / ATT_BT) * ATT_BT;
    const int qend = W > 0 ? min(T, k0 + ATT_BQ - 1 + W) : T;
    for (int qt = qbeg; qt < qend; qt += ATT_BT) {
        __syncthreads();
        stage_rows_major<HD, ATT_BT>(Qs, Q, a.ldq, qt, T);
        stage_cols_major<HD, ATT_BT>(Qt, Q, a.ldq, qt, T);
        stage_rows_major<HD, ATT_BT>(Gs, G, a.lddo, qt, T);
        stage_cols_major<HD, ATT_BT>(Gt, G, a.lddo, qt, T);
        for (int i = threadIdx.x; i < ATT_BT; i += 256) {
            int q = qt + i;
            Ls[i] = q < T ? LSE[q] * M_LOG2E_F : 0.f;
            Ds[i] = q < T ? DD[q] : 0.f;
        }
        __syncthreads();
        if (qt + ATT_BT - 1 < kw) continue;                         // every query precedes every key of the wave
        if (W > 0 && qt > kw + 31 + W - 1) continue;               // every query is past every window
        const bool need_mask = (qt < kw + 31) || (qt + ATT_BT > T) || (W > 0 && qt + ATT_BT - 1 - kw >= W);
        bf16x8 pk[4], dsk[4];
#pragma unroll
        for (int qf = 0; qf < 2; ++qf) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s = mfma(frag_rows<HD>(Qs, qf * 32 + lr, ds, hh), kf[ds], s);
                dp = mfma(frag_rows<HD>(Gs, qf * 32 + lr, ds, hh), vf[ds], dp);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int qi = qf * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                float p = exp2f(fmaf(s[e], c, -Ls[qi]));
                if (need_mask && !visible(qt + qi, mykey, T, W)) p = 0.f;
                const float dsv = p * (dp[e] - Ds[qi]);
                pk[2 * qf + (e >> 3)][e & 7] = (bf16)p;
                dsk[2 * qf + (e >> 3)][e & 7] = (bf16)dsv;
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int df = 0; df < NDF; ++df) {
                dv[df] = mfma(frag_cols<ATT_BT>(Gt, df * 32 + lr, ks, hh), pk[ks], dv[df]);
                dk[df] = mfma(frag_cols<ATT_BT>(Qt, df * 32 + lr, ks, hh), dsk[ks], dk[df]);
            }
    }
    if (mykey < T) {
        const float isd = 1.0f / sqrtf((float)HD);
        bf16* DK = (bf16*)a.dk + ((int64_t)b * T + mykey) * a.ldd + h * HD;
        bf16* DV = (bf16*)a.dv + ((int64_t)b * T + mykey) * a.ldd + h * HD;
#pragma unroll
        for (int df = 0; df < NDF; ++df)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 vk, vv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    vk[i] = (bf16)(dk[df][4 * g4 + i] * isd);
                    vv[i] = (bf16)dv[df][4 * g4 + i];
                }
                *reinterpret_cast<bf16x4*>(DK + df * 32 + 8 * g4 + 4 * hh) = vk;
                *reinterpret_cast<bf16x4*>(DV + df * 32 + 8 * g4 + 4 * hh) = vv;
            }
    }
}

// ============================================================== backward: dQ

template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_dq_mfma_kernel(Attn a) {
    constexpr int NDS = HD / 16, NDF = HD / 32, SK = HD + 8, ST = ATT_BT + 4;
    __shared__ __attribute__((aligned(16))) bf16 Ks[ATT_BT * SK];
    __shared__ __attribute__((aligned(16))) bf16 Kt[HD * ST];
    __shared__ __attribute__((aligned(16))) bf16 Vs[ATT_BT * SK];
    const int qtile = gridDim.x - 1 - blockIdx.x;
    const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
    const int T = a.T, W = a.window;
    const int q0 = qtile * ATT_BQ;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lr = lane & 31, hh = lane >> 5;
    const int qw = q0 + w * 32, myq = qw + lr;
    const bf16* Q = (const bf16*)a.q + (int64_t)b * T * a.ldq + h * HD;
    const bf16* K = (const bf16*)a.k + (int64_t)b * T * a.ldk + h * HD;
    const bf16* V = (const bf16*)a.v + (int64_t)b * T * a.ldv + h * HD;
    const bf16* G = (const bf16*)a.dO + (int64_t)b * T * a.lddo + h * HD;

    bf16x8 qf[NDS], gf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        bf16x8 z = {};
        qf[ds] = myq < T ? load8(Q + (int64_t)myq * a.ldq + 16 * ds + 8 * hh) : z;
        gf[ds] = myq < T ? load8(G + (int64_t)myq * a.lddo + 16 * ds + 8 * hh) : z;
    }
    const float c = M_LOG2E_F / sqrtf((float)HD);
    const float lse2 = myq < T ? a.lse[(int64_t)bh * T + myq] * M_LOG2E_F : 0.f;
    const float Dq = myq < T ? a.D[(int64_t)bh * T + myq] : 0.f;
    f32x16 dq[NDF];
#pragma unroll
    for (int df = 0; df < NDF; ++df) dq[df] = zero16();
    const int kend = min(T, q0 + ATT_BQ);
    int kbeg = W > 0 ? max(0, q0 - W + 1) : 0;
    kbeg = (kbeg / ATT_BT) * ATT_BT;
    for (int kt = kbeg; kt < kend; kt += ATT_BT) {
        __syncthreads();
        stage_rows_major<HD, ATT_BT>(Ks, K, a.ldk, kt, T);
        stage_cols_major<HD, ATT_BT>(Kt, K, a.ldk, kt, T);
        stage_rows_major<HD, ATT_BT>(Vs, V, a.ldv, kt, T);
        __syncthreads();
        if (kt > qw + 31) continue;
        if (W > 0 && kt + ATT_BT - 1 <= qw - W) continue;
        const bool need_mask = (kt + ATT_BT - 1 > qw) || (kt + ATT_BT > T) || (W > 0 && qw + 31 - kt >= W);
        bf16x8 dsk[4];
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s = mfma(frag_rows<HD>(Ks, kf * 32 + lr, ds, hh), qf[ds], s);
                dp = mfma(frag_rows<HD>(Vs, kf * 32 + lr, ds, hh), gf[ds], dp);
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float p = exp2f(fmaf(s[e], c, -lse2));
                if (need_mask) {
                    int key = kt + kf * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                    if (!visible(myq, key, T, W)) p = 0.f;
                }
                dsk[2 * kf + (e >> 3)][e & 7] = (bf16)(p * (dp[e] - Dq));
            }
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int df = 0; df < NDF; ++df)
                dq[df] = mfma(frag_cols<ATT_BT>(Kt, df * 32 + lr, ks, hh), dsk[ks], dq[df]);
    }
    if (myq < T) {
        const float isd = 1.0f / sqrtf((float)HD);
        bf16* DQ = (bf16*)a.dq + ((int64_t)b * T + myq) * a.ldd + h * HD;
#pragma unroll
        for (int df = 0; df < NDF; ++df)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                bf16x4 v;
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = (bf16)(dq[df][4 * g4 + i] * isd);
                *reinterpret_cast<bf16x4*>(DQ + df * 32 + 8 * g4 + 4 * hh) = v;
            }
    }
}

// ============================================================== dispatch

static bool mfma_ok(const Attn& a) {
    if (!a.bf || (a.hd != 64 && a.hd != 128)) return false;
    auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (!al(a.q) || !al(a.k) || !al(a.v)) return false;
    if (a.ldq % 8 || a.ldk % 8 || a.ldv % 8) return false;
    return true;
}

bool attention_fwd_mfma(const Attn& a, hipStream_t s) {
    if (!mfma_ok(a) || a.ldo % 4) return false;
    dim3 grid(ceil_div(a.T, ATT_BQ), a.B * a.H);
    if (a.hd == 64) attn_fwd_mfma_kernel<64><<<grid, 256, 0, s>>>(a);
    else attn_fwd_mfma_kernel<128><<<grid, 256, 0, s>>>(a);
    return true;
}

bool attention_bwd_mfma(const Attn& a, hipStream_t s) {
    if (!mfma_ok(a) || a.lddo % 8 || a.ldd % 4) return false;
    auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (!al(a.dO)) return false;
    dim3 grid(ceil_div(a.T, ATT_BQ), a.B * a.H);
    if (a.hd == 64) {
        attn_bwd_dkdv_mfma_kernel<64><<<grid, 256, 0, s>>>(a);
        attn_bwd_dq_mfma_kernel<64><<<grid, 256, 0, s>>>(a);
    } else {
        attn_bwd_dkdv_mfma_kernel<128><<<grid, 256, 0, s>>>(a);
        attn_bwd_dq_mfma_kernel<128><<<grid, 256, 0, s>>>(a);
    }
    return true;
}

}  // namespace gk
