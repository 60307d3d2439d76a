// Causal multi-head attention, forward and backward, without materialising
// the T x T matrix: O = softmax(Q K^T / sqrt(d_k)) V with Attn_ij = 0 for
// j > i ("NanoGPT Speedrun baseline" (cruxr.ai), "El Mecanismo de Atención"),
// heads as a batch dimension ("Zero to Hero, lecture 9" (ai.flicky.cc),
// "Раздел 1 / Архитектура"), computed block by block with a running maximum
// and a running sum that is rescaled when the maximum grows (the online
// softmax of the "Раздел 2. Сделаем быстро" FlashAttention paragraph).
// An optional window W keeps only keys with i - j < W (the long/short
// sliding windows of the Modded-NanoGPT README).
//
// The forward pass saves LSE_i = log sum_j exp(s_ij); the backward pass
// recomputes P_ij = exp(s_ij - LSE_i) and uses D_i = sum_c dO_ic O_ic:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
//   dQ = dS K / sqrt(d_k),  dK = dS^T Q / sqrt(d_k).
// dQ is produced by one kernel (rows of queries), dK and dV by another (rows of
// keys), so no two workgroups write the same output: no atomics.
//
// This file is the portable FMA version (any head dim in {16, 32, 64, 128},
// fp32 or bf16 storage); attention_mfma.hip holds the matrix-core kernels.
#include "common.h"
#include "kernels.h"

namespace gk {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Group of G = HD/16 consecutive lanes per query (or key) row; each lane owns
// 16 of the head's dimensions.
template <int G>
GPT_DEV float group_sum(float v) {
#pragma unroll
    for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <typename T>
GPT_DEV void load16(const T* p, float* out) {
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
        float4 v = load4(p + e);
        out[e] = v.x; out[e + 1] = v.y; out[e + 2] = v.z; out[e + 3] = v.w;
    }
}
template <typename T>
GPT_DEV void store16(T* p, const float* v) {
#pragma unroll
    for (int e = 0; e < 16; e += 4) store4(p + e, make_float4(v[e], v[e + 1], v[e + 2], v[e + 3]));
}

// Stage `rows` rows of HD values (row stride ld, element offset col) into LDS as fp32.
template <typename T, int HD>
GPT_DEV void stage_rows(float (*dst)[HD + 4], const T* src, int64_t ld, int r0, int rows, int T_, int64_t base) {
    constexpr int V4 = HD / 4;
    for (int i = threadIdx.x; i < rows * V4; i += blockDim.x) {
        int r = i / V4, c = (i % V4) * 4;
        int gr = r0 + r;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (gr < T_) v = load4(src + base + (int64_t)gr * ld + c);
        *reinterpret_cast<float4*>(&dst[r][c]) = v;
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_fwd_simple_kernel(Attn a) {
    constexpr int G = HD / 16, QB = 256 / G, KB = 32;
    __shared__ float Ks[KB][HD + 4];
    __shared__ float Vs[KB][HD + 4];
    const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
    const int T_ = a.T, W = a.window;
    const int q0 = blockIdx.x * QB;
    const int row = q0 + threadIdx.x / G, sub = threadIdx.x % G;
    const T* Q = (const T*)a.q;
    const T* K = (const T*)a.k;
    const T* V = (const T*)a.v;
    const int64_t rowbase = (int64_t)b * T_;
    const float sc = LOG2E / sqrtf((float)HD);
    float q[16], o[16];
    if (row < T_) load16(Q + (rowbase + row) * a.ldq + h * HD + sub * 16, q);
    else for (int e = 0; e < 16; ++e) q[e] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) { q[e] *= sc; o[e] = 0.f; }
    float mx = -INFINITY, l = 0.f;
    const int kend = min(T_, q0 + QB);
    const int kstart = W > 0 ? max(0, q0 - W + 1) : 0;
    for (int kt = kstart; kt < kend; kt += KB) {
        __syncthreads();
        stage_rows<T, HD>(Ks, K, a.ldk, kt, KB, T_, rowbase * a.ldk + h * HD);
        stage_rows<T, HD>(Vs, V, a.ldv, kt, KB, T_, rowbase * a.ldv + h * HD);
        __syncthreads();
        for (int j0 = 0; j0 < KB; j0 += 8) {
            float s[8];
            float cm = -INFINITY;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float* kr = &Ks[j0 + u][sub * 16];
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc = fmaf(q[e], kr[e], acc);
                acc = group_sum<G>(acc);
                int key = kt + j0 + u;
                bool ok = key <= row && key < T_ && (W <= 0 || row - key < W);
                s[u] = ok ? acc : -INFINITY;
                cm = fmaxf(cm, s[u]);
            }
            float mn = fmaxf(mx, cm);
            if (mn == -INFINITY) continue;
            float corr = exp2f(mx - mn);
            l *= corr;
#pragma unroll
            for (int e = 0; e < 16; ++e) o[e] *= corr;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                float p = exp2f(s[u] - mn);
                l += p;
                const float* vr = &Vs[j0 + u][sub * 16];
#pragma unroll
                for (int e = 0; e < 16; ++e) o[e] = fmaf(p, vr[e], o[e]);
            }
            mx = mn;
        }
    }
    if (row < T_) {
        float inv = 1.0f / l;
#pragma unroll
        for (int e = 0; e < 16; ++e) o[e] *= inv;
        store16((T*)a.o + (rowbase + row) * a.ldo + h * HD + sub * 16, o);
        if (sub == 0) a.lse[(int64_t)bh * T_ + row] = (mx + log2f(l)) * LN2;
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_dq_simple_kernel(Attn a) {
    constexpr int G = HD / 16, QB = 256 / G, KB = 32;
    __shared__ float Ks[KB][HD + 4];
    __shared__ float Vs[KB][HD + 4];
    const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
    const int T_ = a.T, W = a.window;
    const int q0 = blockIdx.x * QB;
    const int row = q0 + threadIdx.x / G, sub = threadIdx.x % G;
    const int64_t rowbase = (int64_t)b * T_;
    const float isd = 1.0f / sqrtf((float)HD);
    float q[16], dO[16], dq[16];
    float lse2 = 0.f, Di = 0.f;
    if (row < T_) {
        load16((const T*)a.q + (rowbase + row) * a.ldq + h * HD + sub * 16, q);
        load16((const T*)a.dO + (rowbase + row) * a.lddo + h * HD + sub * 16, dO);
        lse2 = a.lse[(int64_t)bh * T_ + row] * LOG2E;
        Di = a.D[(int64_t)bh * T_ + row];
    } else {
        for (int e = 0; e < 16; ++e) q[e] = dO[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) { q[e] *= isd * LOG2E; dq[e] = 0.f; }
    const int kend = min(T_, q0 + QB);
    const int kstart = W > 0 ? max(0, q0 - W + 1) : 0;
    for (int kt = kstart; kt < kend; kt += KB) {
        __syncthreads();
        stage_rows<T, HD>(Ks, (const T*)a.k, a.ldk, kt, KB, T_, rowbase * a.ldk + h * HD);
        stage_rows<T, HD>(Vs, (const T*)a.v, a.ldv, kt, KB, T_, rowbase * a.ldv + h * HD);
        __syncthreads();
        for (int j = 0; j < KB; ++j) {
            const float* kr = &Ks[j][sub * 16];
            const float* vr = &Vs[j][sub * 16];
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) { s = fmaf(q[e], kr[e], s); dp = fmaf(dO[e], vr[e], dp); }
            s = group_sum<G>(s);
            dp = group_sum<G>(dp);
            int key = kt + j;
            bool ok = row < T_ && key <= row && (W <= 0 || row - key < W);
            float p = ok ? exp2f(s - lse2) : 0.f;
            float ds = p * (dp - Di);
#pragma unroll
            for (int e = 0; e < 16; ++e) dq[e] = fmaf(ds, kr[e], dq[e]);
        }
    }
    if (row < T_) {
#pragma unroll
        for (int e = 0; e < 16; ++e) dq[e] *= isd;
        store16((T*)a.dq + (rowbase + row) * a.ldd + h * HD + sub * 16, dq);
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_simple_kernel(Attn a) {
    constexpr int G = HD / 16, KR = 256 / G, QT = 32;
    __shared__ float Qs[QT][HD + 4];
    __shared__ float dOs[QT][HD + 4];
    __shared__ float Ls[QT], Ds[QT];
    const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
    const int T_ = a.T, W = a.window;
    const int k0 = blockIdx.x * KR;
    const int key = k0 + threadIdx.x / G, sub = threadIdx.x % G;
    const int64_t rowbase = (int64_t)b * T_;
    const float isd = 1.0f / sqrtf((float)HD);
    float k[16], v[16], dk[16], dv[16];
    if (key < T_) {
        load16((const T*)a.k + (rowbase + key) * a.ldk + h * HD + sub * 16, k);
        load16((const T*)a.v + (rowbase + key) * a.ldv + h * HD + sub * 16, v);
    } else {
        for (int e = 0; e < 16; ++e) k[e] = v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) { k[e] *= isd * LOG2E; dk[e] = dv[e] = 0.f; }
    const int qstart = k0;
    const int qend = W > 0 ? min(T_, k0 + KR - 1 + W) : T_;
    for (int qt = qstart; qt < qend; qt += QT) {
        __syncthreads();
        stage_rows<T, HD>(Qs, (const T*)a.q, a.ldq, qt, QT, T_, rowbase * a.ldq + h * HD);
        stage_rows<T, HD>(dOs, (const T*)a.dO, a.lddo, qt, QT, T_, rowbase * a.lddo + h * HD);
        for (int i = threadIdx.x; i < QT; i += blockDim.x) {
            int gq = qt + i;
            Ls[i] = gq < T_ ? a.lse[(int64_t)bh * T_ + gq] * LOG2E : 0.f;
            Ds[i] = gq < T_ ? a.D[(int64_t)bh * T_ + gq] : 0.f;
        }
        __syncthreads();
        for (int i = 0; i < QT; ++i) {
            const float* qr = &Qs[i][sub * 16];
            const float* gr = &dOs[i][sub * 16];
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) { s = fmaf(qr[e], k[e], s); dp = fmaf(gr[e], v[e], dp); }
            s = group_sum<G>(s);
            dp = group_sum<G>(dp);
            int qi = qt + i;
            bool ok = key < T_ && qi < T_ && key <= qi && (W <= 0 || qi - key < W);
            float p = ok ? exp2f(s - Ls[i]) : 0.f;
            float ds = p * (dp - Ds[i]);
#pragma unroll
            for (int e = 0; e < 16; ++e) { dv[e] = fmaf(p, gr[e], dv[e]); dk[e] = fmaf(ds, qr[e], dk[e]); }
        }
    }
    if (key < T_) {
#pragma unroll
        for (int e = 0; e < 16; ++e) dk[e] *= isd;
        store16((T*)a.dk + (rowbase + key) * a.ldd + h * HD + sub * 16, dk);
        store16((T*)a.dv + (rowbase + key) * a.ldd + h * HD + sub * 16, dv);
    }
}

template <typename T, int HD>
static void fwd_simple(const Attn& a, hipStream_t s) {
    constexpr int QB = 256 / (HD / 16);
    dim3 grid(ceil_div(a.T, QB), a.B * a.H);
    attn_fwd_simple_kernel<T, HD><<<grid, 256, 0, s>>>(a);
}
template <typename T, int HD>
static void bwd_simple(const Attn& a, hipStream_t s) {
    constexpr int QB = 256 / (HD / 16);
    dim3 grid(ceil_div(a.T, QB), a.B * a.H);
    attn_bwd_dq_simple_kernel<T, HD><<<grid, 256, 0, s>>>(a);
    attn_bwd_dkdv_simple_kernel<T, HD><<<grid, 256, 0, s>>>(a);
}

template <typename T>
static void fwd_simple_t(const Attn& a, hipStream_t s) {
    switch (a.hd) {
        case 16: fwd_simple<T, 16>(a, s); break;
        case 32: fwd_simple<T, 32>(a, s); break;
        case 64: fwd_simple<T, 64>(a, s); break;
        case 128: fwd_simple<T, 128>(a, s); break;
    }
}
template <typename T>
static void bwd_simple_t(const Attn& a, hipStream_t s) {
    switch (a.hd) {
        case 16: bwd_simple<T, 16>(a, s); break;
        case 32: bwd_simple<T, 32>(a, s); break;
        case 64: bwd_simple<T, 64>(a, s); break;
        case 128: bwd_simple<T, 128>(a, s); break;
    }
}

void attention_fwd_simple(const Attn& a, hipStream_t s) {
    if (a.bf) fwd_simple_t<bf16>(a, s);
    else fwd_simple_t<float>(a, s);
}
void attention_bwd_simple(const Attn& a, hipStream_t s) {
    if (a.bf) bwd_simple_t<bf16>(a, s);
    else bwd_simple_t<float>(a, s);
}

bool attention_fwd_mfma(const Attn& a, hipStream_t s);
bool attention_bwd_mfma(const Attn& a, hipStream_t s);

void attention_fwd(const Attn& a, hipStream_t s) {
    if (!attention_fwd_mfma(a, s)) attention_fwd_simple(a, s);
}
bool attention_bwd(const Attn& a, hipStream_t s) {
    if (attention_bwd_mfma(a, s)) return true;
    attn_rowdot(a.bf, a.dO, a.o, a.Dout, a.B, a.T, a.H, a.hd, s);
    attention_bwd_simple(a, s);
    return false;
}

}  // namespace gk
