// bf16 matrix-core GEMM for gfx950 (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
// with the fused epilogues of gemm_common.h. Used for every linear-layer
// product of the bf16 training step (the bf16 autocast matmuls of the
// lecture notes' "Раздел 2. Сделаем быстро", rebuilt for CDNA4).
//
// Structure
//   * 256 threads = 4 wavefronts in a WGM x WGN grid; each wavefront owns a
//     (BM/WGM) x (BN/WGN) sub-tile made of 32x32 MFMA fragments.
//   * Both operands are staged through LDS as [row][k] tiles (row = m for A,
//     n for B) so that every lane reads its 8 consecutive k values of a
//     fragment with one 16-byte LDS read. Rows are padded by 16 bytes and the
//     16-byte chunks of a row are XOR-swizzled by (row / 8) to keep both the
//     writes and the fragment reads free of bank conflicts.
//   * Operands stored k-contiguous in memory (activations X and weights W of
//     X W^T) are copied in 16-byte chunks. Operands stored row-contiguous
//     (the dY and X of dW = dY^T X, and W in dX = dY W) are read as two
//     16-byte rows (k, k+1) of 8 consecutive rows each, and written to LDS as
//     eight 4-byte (k, k+1) pairs: the transposition happens in registers.
//   * Two LDS buffers: the next k-tile is fetched from global memory into
//     registers while the current one feeds the matrix cores.
//   * Split-K (grid.z) writes fp32 partial tiles; a second kernel sums the
//     slices in a fixed order and applies the epilogue (deterministic).
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace gk {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

GPT_DEV int swz(int row, int kc, int ch) { return kc ^ ((row >> 3) & (ch - 1)); }

template <int R, int BK>
struct DirectTile {   // element (r, k) at base[r * ld + k]
    static constexpr int CH = BK / 8, NCH = R * CH, PER = (NCH + 255) / 256, S = BK + 8;
    u32x4 reg[PER];
    GPT_DEV void load(const bf16* base, int64_t ld, int row0, int rows, int k0, int K) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            int c = threadIdx.x + 256 * p;
            int r = c / CH, kc = c % CH;
            int gr = row0 + r, gk = k0 + kc * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if ((NCH % 256 == 0 || c < NCH) && gr < rows && gk < K)
                v = *reinterpret_cast<const u32x4*>(base + (int64_t)gr * ld + gk);
            reg[p] = v;
        }
    }
    GPT_DEV void store(bf16* lds) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            int c = threadIdx.x + 256 * p;
            if (NCH % 256 != 0 && c >= NCH) continue;
            int r = c / CH, kc = c % CH;
            *reinterpret_cast<u32x4*>(lds + r * S + swz(r, kc, CH) * 8) = reg[p];
        }
    }
};

template <int R, int BK>
struct TransTile {    // element (r, k) at base[k * ld + r]; rows % 8 == 0
    static constexpr int CH = BK / 8, RG = R / 8, KP = BK / 2, NU = RG * KP, PER = (NU + 255) / 256, S = BK + 8;
    u32x4 reg[PER][2];
    GPT_DEV void load(const bf16* base, int64_t ld, int row0, int rows, int k0, int K) {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            int u = threadIdx.x + 256 * p;
            int rg = u % RG, kp = u / RG;
            int gr = row0 + rg * 8, gk = k0 + 2 * kp;
            u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
            if ((NU % 256 == 0 || u < NU) && gr < rows) {
                if (gk < K) v0 = *reinterpret_cast<const u32x4*>(base + (int64_t)gk * ld + gr);
                if (gk + 1 < K) v1 = *reinterpret_cast<const u32x4*>(base + (int64_t)(gk + 1) * ld + gr);
            }
            reg[p][0] = v0;
            reg[p][1] = v1;
        }
    }
    GPT_DEV void store(bf16* lds) const {
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            int u = threadIdx.x + 256 * p;
            if (NU % 256 != 0 && u >= NU) continue;
            int rg = u % RG, kp = u / RG;
            int k = 2 * kp, kc = k >> 3, ko = k & 7;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                uint32_t lo = (reg[p][0][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                uint32_t hi = (reg[p][1][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                int r = rg * 8 + i;
                *reinterpret_cast<uint32_t*>(lds + r * S + swz(r, kc, CH) * 8 + ko) = lo | (hi << 16);
            }
        }
    }
};

template <int R, int BK, bool KC>
using Tile = typename std::conditional<KC, DirectTile<R, BK>, TransTile<R, BK>>::type;

// SPLIT: write fp32 partial sums to part[z][M][N] instead of the epilogue.
template <int BM, int BN, int BK, int WGM, int WGN, bool AKC, bool BKC, int EPI, typename TC, bool SPLIT>
__global__ __launch_bounds__(256, 1) void gemm_mfma_kernel(Gemm g, int kps, float* part) {
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32, S = BK + 8, CH = BK / 8;
    extern __shared__ __attribute__((aligned(16))) char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);
    bf16* As[2] = {smem, smem + (BM + BN) * S};
    bf16* Bs[2] = {smem + BM * S, smem + (BM + BN) * S + BM * S};

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int wm = (w / WGN) * WM, wn = (w % WGN) * WN;
    const int kb = blockIdx.z * kps;
    const int ke = min(g.K, kb + kps);
    const bf16* A = (const bf16*)g.A;
    const bf16* B = (const bf16*)g.B;

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    Tile<BM, BK, AKC> ta;
    Tile<BN, BK, BKC> tb;
    ta.load(A, g.lda, m0, g.M, kb, ke);
    tb.load(B, g.ldb, n0, g.N, kb, ke);
    ta.store(As[0]);
    tb.store(Bs[0]);
    __syncthreads();
    int buf = 0;
    const int lr = lane & 31, lk = lane >> 5;
    for (int k0 = kb; k0 < ke; k0 += BK) {
        const bool more = k0 + BK < ke;
        if (more) {
            ta.load(A, g.lda, m0, g.M, k0 + BK, ke);
            tb.load(B, g.ldb, n0, g.N, k0 + BK, ke);
        }
        const bf16* as = As[buf];
        const bf16* bs = Bs[buf];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 a[FM], b[FN];
            const int kc = kk * 2 + lk;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                int r = wm + i * 32 + lr;
                a[i] = *reinterpret_cast<const bf16x8*>(as + r * S + swz(r, kc, CH) * 8);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                int r = wn + j * 32 + lr;
                b[j] = *reinterpret_cast<const bf16x8*>(bs + r * S + swz(r, kc, CH) * 8);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (more) {
            ta.store(As[buf ^ 1]);
            tb.store(Bs[buf ^ 1]);
        }
        __syncthreads();
        buf ^= 1;
    }
    // accumulator fragment: lane holds column (lane % 32), rows 8*(e/4) + 4*(lane/32) + e%4
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn + j * 32 + lr;
            if (col >= g.N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm + i * 32 + 8 * (e >> 2) + 4 * lk + (e & 3);
                if (row >= g.M) continue;
                if constexpr (SPLIT) part[((int64_t)blockIdx.z * g.M + row) * g.N + col] = acc[i][j][e];
                else epilogue_store<TC, EPI>(g, row, col, acc[i][j][e]);
            }
        }
}

template <typename TC, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(Gemm g, const float* part, int splits) {
    int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    int64_t mn = (int64_t)g.M * g.N;
    if (idx >= mn) return;
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += part[z * mn + idx];
    epilogue_store<TC, EPI>(g, (int)(idx / g.N), (int)(idx % g.N), s);
}

// ------------------------------------------------------------------ dispatch

template <int BM, int BN, int BK, int WGM, int WGN, bool AKC, bool BKC>
struct Launcher {
    static constexpr size_t LDS = (size_t)2 * (BM + BN) * (BK + 8) * sizeof(bf16);

    template <int EPI, typename TC, bool SPLIT>
    static void go(const Gemm& g, dim3 grid, int kps, float* part, hipStream_t s) {
        auto k = gemm_mfma_kernel<BM, BN, BK, WGM, WGN, AKC, BKC, EPI, TC, SPLIT>;
        static bool attr = false;
        if (!attr) {
            (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS);
            attr = true;
        }
        k<<<grid, 256, LDS, s>>>(g, kps, part);
    }

    static void run(const Gemm& g, int splits, float* part, hipStream_t s) {
        dim3 grid(ceil_div(g.N, BN), ceil_div(g.M, BM), splits);
        int kps = ceil_div(ceil_div(g.K, splits), BK) * BK;
        if (splits > 1) {
            go<EPI_STORE, float, true>(g, grid, kps, part, s);
            int64_t mn = (int64_t)g.M * g.N;
            unsigned rb = (unsigned)((mn + 255) / 256);
            switch (g.epi) {
                case EPI_STORE:
                    if (g.c_bf) splitk_reduce_kernel<bf16, EPI_STORE><<<rb, 256, 0, s>>>(g, part, splits);
                    else splitk_reduce_kernel<float, EPI_STORE><<<rb, 256, 0, s>>>(g, part, splits);
                    break;
                case EPI_BIAS: splitk_reduce_kernel<bf16, EPI_BIAS><<<rb, 256, 0, s>>>(g, part, splits); break;
                case EPI_BIAS_ACT: splitk_reduce_kernel<bf16, EPI_BIAS_ACT><<<rb, 256, 0, s>>>(g, part, splits); break;
                case EPI_BIAS_RESID: splitk_reduce_kernel<float, EPI_BIAS_RESID><<<rb, 256, 0, s>>>(g, part, splits); break;
                case EPI_ACT_GRAD: splitk_reduce_kernel<bf16, EPI_ACT_GRAD><<<rb, 256, 0, s>>>(g, part, splits); break;
                case EPI_ACCUM: splitk_reduce_kernel<float, EPI_ACCUM><<<rb, 256, 0, s>>>(g, part, splits); break;
            }
            return;
        }
        switch (g.epi) {
            case EPI_STORE:
                if (g.c_bf) go<EPI_STORE, bf16, false>(g, grid, kps, part, s);
                else go<EPI_STORE, float, false>(g, grid, kps, part, s);
                break;
            case EPI_BIAS: go<EPI_BIAS, bf16, false>(g, grid, kps, part, s); break;
            case EPI_BIAS_ACT: go<EPI_BIAS_ACT, bf16, false>(g, grid, kps, part, s); break;
            case EPI_BIAS_RESID: go<EPI_BIAS_RESID, float, false>(g, grid, kps, part, s); break;
            case EPI_ACT_GRAD: go<EPI_ACT_GRAD, bf16, false>(g, grid, kps, part, s); break;
            case EPI_ACCUM: go<EPI_ACCUM, float, false>(g, grid, kps, part, s); break;
        }
    }
};

template <bool AKC, bool BKC>
static void run_layout(const Gemm& g, float* scratch, size_t nscratch, hipStream_t s) {
    const int64_t t256 = (int64_t)ceil_div(g.M, 256) * ceil_div(g.N, 256);
    const int64_t t128 = (int64_t)ceil_div(g.M, 128) * ceil_div(g.N, 128);
    const int64_t mn = (int64_t)g.M * g.N;
    // fill the 256 compute units: large tiles when there are enough of them,
    // otherwise 128x128, and split K when even those leave the chip idle
    if (t256 >= 240) {
        Launcher<256, 256, 32, 2, 2, AKC, BKC>::run(g, 1, nullptr, s);
        return;
    }
    int splits = 1;
    if (t128 < 200 && g.K >= 2048 && scratch) {
        splits = (int)std::min<int64_t>(16, (512 + t128 - 1) / t128);
        while (splits > 1 && ((size_t)splits * mn > nscratch || g.K / splits < 256)) --splits;
    }
    Launcher<128, 128, 32, 2, 2, AKC, BKC>::run(g, splits, scratch, s);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool gemm_mfma_ok(const Gemm& g) {
    if (!g.in_bf || g.K % 8) return false;
    if (!aligned16(g.A) || !aligned16(g.B)) return false;
    if (g.lda % 8 || g.ldb % 8) return false;
    if (!g.a_kc && g.M % 8) return false;
    if (!g.b_kc && g.N % 8) return false;
    if (!g.a_kc && g.b_kc) return false;     // orientation not used by the training step
    return true;
}

void gemm_mfma(const Gemm& g, float* scratch, size_t nscratch, hipStream_t s) {
    if (g.a_kc && g.b_kc) run_layout<true, true>(g, scratch, nscratch, s);
    else if (g.a_kc) run_layout<true, false>(g, scratch, nscratch, s);
    else run_layout<false, false>(g, scratch, nscratch, s);
}

}  // namespace gk
