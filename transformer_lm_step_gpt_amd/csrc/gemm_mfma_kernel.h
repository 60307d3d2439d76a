// bf16 matrix-core GEMM kernel for gfx950 (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
// with the fused epilogues of gemm_common.h. Used for every linear-layer
// product of the bf16 training step (the bf16 autocast matmuls of the
// lecture notes' "Раздел 2. Сделаем быстро", rebuilt for CDNA4).
//
// Structure
//   * 4 or 8 wavefronts in a WGM x WGN grid; each wavefront owns a
//     (BM/WGM) x (BN/WGN) sub-tile made of 32x32 MFMA fragments.
//   * Global -> LDS copies either use the 16-byte LDS-DMA load (each lane's
//     16 bytes land at LDS base + 16 * lane), so no registers are spent on
//     staging, and a k-tile is copied as soon as its stage is free (a ring of
//     NS LDS stages; a k-tile is waited for with s_waitcnt vmcnt only when
//     consumed), or go through registers (16-byte buffer loads one k-tile
//     ahead, ds_write_b128 into the same LDS layout): see PIPE below.
//   * An operand stored k-contiguous (X and W of X W^T) is kept as a
//     [row][BK] tile; a fragment (8 consecutive k of one row per lane) is one
//     16-byte LDS read.
//   * An operand stored row-contiguous (dY and X of dW = dY^T X, W of
//     dX = dY W) is kept as it is in memory, a [BK][rows] tile; fragments are
//     built with the transposing LDS read ds_read_b64_tr_b16: in each group of
//     16 lanes, lane j addresses 4 consecutive rows of k-row k0 + j/4 and lane
//     i receives k0..k0+3 of row i. Two such reads give the 8 k values.
//   * 16-byte chunks of every LDS row are XOR-swizzled (by the row index for
//     [row][BK] tiles, by the k index for [BK][rows] tiles); the DMA lanes
//     pick the global chunk that belongs at their LDS slot, so both the
//     copies and the fragment reads avoid bank conflicts.
//   * Split-K (grid.z) writes fp32 partial tiles; a second kernel sums the
//     slices in a fixed order and applies the epilogue (deterministic).
//   * Workgroup i (flattened over the split-K slices) runs on XCD i % 8; the
//     work items (k-slice, output tile) are renumbered so that each XCD owns
//     a contiguous range of them, slice by slice and tiles in a grouped order
//     (bands of 8 tile-rows walked column by column), so the A and B panels
//     of the items in flight on one XCD stay in its L2.
#pragma once
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

#include <type_traits>

namespace gk {

namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int s32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// s_waitcnt with vmcnt <= n and the other counters unconstrained (gfx9 encoding)
template <int N>
GPT_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the release fence of __syncthreads (which would
// wait for every in-flight LDS-DMA load). Each wave has already waited, with
// s_waitcnt vmcnt, for the DMA loads of the tile it is about to read; after
// the barrier every wave's loads of that tile are complete.
GPT_DEV void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

GPT_DEV void dma16(const void* g, bf16* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds_wave_base, 16, 0, 0);
}

// ---- [row][BK] tile of an operand stored k-contiguous (element (r, k) at base[r * ld + k])
template <int R, int BK, int NW>
struct RowTile {
    static constexpr int CH = BK / 8;                 // 16-byte chunks per row
    static constexpr int ROWS_PER_DMA = 64 / CH;      // rows filled by one wave-wide DMA (1 KiB)
    static constexpr int DMAS = R / ROWS_PER_DMA;     // per tile
    static constexpr int PER_WAVE = DMAS / NW;
    static constexpr int BYTES = R * BK * 2;
    static constexpr int READS_PER_FRAG = 1;
    static_assert(DMAS % NW == 0, "tile too small for the waves");
    GPT_DEV static int swz(int r) { return CH == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
    // per-lane sources of this wave's DMAs for rows [row0, row0 + R), k [k0, k0 + BK);
    // each later k-tile is STEP elements further on
    GPT_DEV static void src_init(const bf16* (&src)[PER_WAVE], const bf16* base, int64_t ld, int row0, int rows, int k0,
                                 int w, int lane) {
#pragma unroll
        for (int p = 0; p < PER_WAVE; ++p) {
            const int d = w * PER_WAVE + p;
            const int r = d * ROWS_PER_DMA + lane / CH;
            const int kc = (lane % CH) ^ swz(r);
            const int gr = min(row0 + r, rows - 1);    // rows past the end feed only unstored outputs
            src[p] = base + (int64_t)gr * ld + k0 + kc * 8;
        }
    }
    GPT_DEV static int64_t step(int64_t) { return BK; }
    // 8 consecutive k (16*ks + 8*hk ...) of row r
    GPT_DEV static bf16x8 frag(const bf16* tile, int r, int ks, int hk) {
        const int kc = 2 * ks + hk;
        return *reinterpret_cast<const bf16x8*>(tile + r * BK + ((kc ^ swz(r)) << 3));
    }
};

// ---- [BK][row] tile of an operand stored row-contiguous (element (r, k) at base[k * ld + r])
template <int R, int BK, int NW>
struct ColTile {
    static constexpr int CH = R / 8;                  // 16-byte chunks per k-row
    static constexpr int DMAS = BK * CH / 64;         // wave-wide 1 KiB copies per tile
    static constexpr int PER_WAVE = DMAS / NW;
    static constexpr int BYTES = R * BK * 2;
    static constexpr int READS_PER_FRAG = 2;
    static_assert(CH >= 16 && CH % 8 == 0 && (BK * CH) % (64 * NW) == 0, "unsupported tile");
    // chunk c of k-row k sits at slot lds_slot(k, c), so that the 4 k-rows x 4
    // chunks a half-wave's transposing read touches fall in 16 different
    // 16-byte bank groups (64 banks): for power-of-two rows (k-rows start at the
    // same bank) an XOR of the chunk's quad with k & 3; for rows of 8 mod 16
    // chunks (odd and even k-rows already half a bank cycle apart) an XOR of
    // the quad with bit 1 of k (an involution, so the same map both ways)
    static constexpr bool POW2 = (CH & (CH - 1)) == 0;
    static_assert(POW2 || CH % 16 == 8, "unsupported row width");
    GPT_DEV static int lds_slot(int k, int c) { return POW2 ? (c ^ ((k & 3) << 2)) : (c ^ ((k & 2) << 1)); }
    GPT_DEV static int glob_chunk(int k, int slot) { return lds_slot(k, slot); }
    GPT_DEV static void src_init(const bf16* (&src)[PER_WAVE], const bf16* base, int64_t ld, int row0, int rows, int k0,
                                 int w, int lane) {
#pragma unroll
        for (int p = 0; p < PER_WAVE; ++p) {
            const int q = (w * PER_WAVE + p) * 64 + lane;   // 16-byte LDS slot this lane fills
            const int k = q / CH;
            const int c = glob_chunk(k, q % CH);
            const int gr = min(row0 + c * 8, rows - 8);   // rows % 8 == 0
            src[p] = base + (int64_t)(k0 + k) * ld + gr;
        }
    }
    GPT_DEV static int64_t step(int64_t ld) { return BK * ld; }
    GPT_DEV static s16x4 tr_read(const bf16* tile, int k, int r) {
        const bf16* p = tile + k * R + (lds_slot(k, r >> 3) << 3) + (r & 7);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
    }
    // fragment of rows rb..rb+31: lane l gets k = 16*ks + 8*(l/32) + e of row rb + l%32
    GPT_DEV static bf16x8 frag(const bf16* tile, int rb, int ks, int lane) {
        const int g = lane >> 4, j = lane & 15;
        const int r = rb + 16 * (g & 1) + 4 * (j & 3);
        const int k = 16 * ks + 8 * (g >> 1) + (j >> 2);
        s16x4 lo = tr_read(tile, k, r);
        s16x4 hi = tr_read(tile, k + 4, r);
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        u32x4 v = {l2[0], l2[1], h2[0], h2[1]};
        return __builtin_bit_cast(bf16x8, v);
    }
};

template <bool KC, int R, int BK, int NW>
struct OpTile;
template <int R, int BK, int NW>
struct OpTile<true, R, BK, NW> : RowTile<R, BK, NW> {
    GPT_DEV static bf16x8 get(const bf16* t, int rb, int ks, int lane) {
        return RowTile<R, BK, NW>::frag(t, rb + (lane & 31), ks, lane >> 5);
    }
};
template <int R, int BK, int NW>
struct OpTile<false, R, BK, NW> : ColTile<R, BK, NW> {
    GPT_DEV static bf16x8 get(const bf16* t, int rb, int ks, int lane) { return ColTile<R, BK, NW>::frag(t, rb, ks, lane); }
};

}  // namespace

// One 16-deep step: the FM x FN products of (ca, cb), with the fragment reads
// of the next step (into na, nb) and the operations of `extra` (slot p runs
// after product p) placed between them in program order, so LDS latency and
// DMA issue hide under the matrix cores.
template <int FM, int FN, class TA, class TB, class X>
__device__ __attribute__((always_inline)) inline void half_step(f32x16 (&acc)[FM][FN], const bf16x8 (&ca)[FM],
                                                               const bf16x8 (&cb)[FN], bf16x8 (&na)[FM],
                                                               bf16x8 (&nb)[FN], const bf16* as, const bf16* bs, int wm,
                                                               int wn, int ksn, int lane, X&& extra) {
    constexpr int NF = FM + FN, P = FM * FN;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        acc[p / FN][p % FN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[p / FN], cb[p % FN], acc[p / FN][p % FN], 0, 0, 0);
        // the next step's fragment reads go out early (one after each of the
        // first NF products), leaving the remaining products to cover their latency
        if (p < NF) {
            const int f = p;
            if (f < FM) na[f] = TA::get(as, wm + 32 * f, ksn, lane);
            else nb[f - FM] = TB::get(bs, wn + 32 * (f - FM), ksn, lane);
        }
        extra(p);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The FM x FN products of one 16-deep step with the operations of `extra`
// (slot p runs after product p) between them in program order.
template <int FM, int FN, class X>
__device__ __attribute__((always_inline)) inline void products(f32x16 (&acc)[FM][FN], const bf16x8 (&ca)[FM],
                                                              const bf16x8 (&cb)[FN], X&& extra) {
    constexpr int P = FM * FN;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        acc[p / FN][p % FN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[p / FN], cb[p % FN], acc[p / FN][p % FN], 0, 0, 0);
        extra(p);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// One 64-deep step on e4m3 operands: the FM x FN products of
// v_mfma_f32_32x32x64_f8f6f4 (32 bytes of A and of B per lane), with the
// operations of `extra` between them in program order.
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <int FM, int FN, class X>
__device__ __attribute__((always_inline)) inline void products_f8(f32x16 (&acc)[FM][FN], const i32x8 (&ca)[FM],
                                                                 const i32x8 (&cb)[FN], X&& extra) {
    constexpr int P = FM * FN;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        acc[p / FN][p % FN] =
            __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ca[p / FN], cb[p % FN], acc[p / FN][p % FN], 0, 0, 0, 0, 0, 0);
        extra(p);
        __builtin_amdgcn_sched_barrier(0);
    }
}

constexpr int GROUP_M = 8;
enum { PIPE_DMA = 0, PIPE_DMA_RS = 1, PIPE_VGPR = 2, PIPE_F8 = 3 };

// SPLIT: write fp32 partial sums to part[z][M][N] instead of the epilogue.
// OUTBF: output storage bf16 (1) or fp32 (0); ACT: activation of the
// BIAS_ACT / ACT_GRAD epilogues. N and ldc are multiples of 8 and the output,
// aux, residual and bias buffers 16-byte aligned (gemm_mfma_ok).
// PIPE (how k-tiles reach LDS and registers):
//   PIPE_DMA: LDS-DMA copies; each 16-deep step's fragments are read during
//     the previous step.
//   PIPE_DMA_RS (register-staged): LDS-DMA copies; a whole k-tile's fragments
//     are read into registers at the start of the tile, so its LDS stage is
//     refilled one step into the tile instead of at its end (each copy has
//     about 1.5 k-tiles of products to land instead of one).
//   PIPE_F8: e4m3 operands (one byte per element, K and the strides counted
//     in 2-byte units, so a 64-unit k-tile holds 128 values) with LDS-DMA
//     copies and register-staged fragments, two 64-deep fp8 products per
//     k-tile; the store epilogue multiplies by out_scale[0] * out_scale[1].
//   PIPE_VGPR: two LDS stages; the copy of k-tile t+2 is loaded into
//     registers (16 bytes per lane per copy) while tile t is multiplied, and
//     written to LDS with ds_write_b128 during tile t+1, so global-load
//     latency has a whole k-tile of products to hide under and the LDS sees
//     ordinary 16-byte writes instead of DMA traffic.
// WGM x WGN waves (4 or 8), each owning a (BM/WGM) x (BN/WGN) sub-tile.
template <int BM, int BN, int BK, int NS, int OCC, int PIPE, int WGM, int WGN, bool AKC, bool BKC, int EPI, int OUTBF,
          int ACT, bool SPLIT>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void gemm_mfma_kernel(Gemm g, int kps, float* part) {
    constexpr bool RS = PIPE == PIPE_DMA_RS;
    using TC = typename std::conditional<OUTBF != 0, bf16, float>::type;
    constexpr int NW = WGM * WGN, NT = 64 * NW;
    constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
    static_assert(FM >= 1 && FN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave sub-tile of 32x32 fragments");
    using TA = OpTile<AKC, BM, BK, NW>;
    using TB = OpTile<BKC, BN, BK, NW>;
    constexpr int STAGE = (TA::BYTES + TB::BYTES) / 2;      // bf16 elements per stage
    constexpr int LPT = TA::PER_WAVE + TB::PER_WAVE;        // DMAs per lane per stage
    static_assert(NS >= 2 && NS <= 4, "stages");
    extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
    bf16* smem = reinterpret_cast<bf16*>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int tn = ceil_div(g.N, BN), tm = ceil_div(g.M, BM), ntiles = tn * tm;
    // XCD-aware renumbering: workgroups are dispatched in order of the
    // flattened id lin = x + ntiles * z, workgroup lin runs on XCD lin % 8, and
    // XCD x takes a contiguous range of the work items (k-slice or batch
    // entry, tile) numbered slice by slice, tiles in the grouped order below. So one XCD's items
    // cover one or two k-slices and a compact group of tiles inside each: its
    // L2 fetches the operand panels of those slices once instead of every
    // slice's whole dY^T panel.
    const int nitems = ntiles * (int)gridDim.z;
    const int lin = blockIdx.x + ntiles * blockIdx.z, xcd = lin & 7, q8 = nitems >> 3, r8 = nitems & 7;
    const int item = xcd * q8 + min(xcd, r8) + (lin >> 3);
    int kz = item / ntiles;
    const int tile = item - kz * ntiles;
    const bf16* A = (const bf16*)g.A;
    const bf16* B = (const bf16*)g.B;
    if constexpr (!SPLIT && EPI == EPI_STORE) {
        if (g.batch > 1) {   // batched product: z is the batch entry, each over the whole K
            A += kz * g.sa;
            B += kz * g.sb;
            g.C = (TC*)g.C + kz * g.sc;
            kz = 0;
        }
    }
    // grouped order: bands of GROUP_M tile-rows, column by column inside a
    // band, so the tiles resident on one XCD at a time share a few A and B
    // panels in its L2
    const int band = tile / (GROUP_M * tn), first = band * GROUP_M, bsz = min(tm - first, GROUP_M);
    const int inb = tile - band * GROUP_M * tn;
    const int m0 = (first + inb % bsz) * BM, n0 = (inb / bsz) * BN;
    const int wm = (w / WGN) * WM, wn = (w % WGN) * WN;
    const int kb = kz * kps;
    const int nk = max(0, (min(g.K, kb + kps) - kb) / BK);    // K and kps are multiples of BK

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // LDS-DMA sources: this wave's PA + PB 16-byte-per-lane copies per k-tile
    constexpr int PA = TA::PER_WAVE, PB = TB::PER_WAVE;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const bf16* srcA[PA];
    const bf16* srcB[PB];
    TA::src_init(srcA, A, g.lda, m0, g.M, kb, wu, lane);
    TB::src_init(srcB, B, g.ldb, n0, g.N, kb, wu, lane);
    const int64_t stA = TA::step(g.lda), stB = TB::step(g.ldb);
    // q-th copy of this wave for the k-tile going into stage st
    auto dma = [&](int q, bf16* st) {
        if (q < PA) {
            dma16(srcA[q], st + (wu * PA + q) * 512);
            srcA[q] += stA;
        } else {
            dma16(srcB[q - PA], st + TA::BYTES / 2 + (wu * PB + q - PA) * 512);
            srcB[q - PA] += stB;
        }
    };

    int issued = 0;   // tiles 0 .. issued-1 have been handed to the LDS-DMA engine
    // wait until tile u is in LDS for every wave: at most (tiles issued after u) x LPT DMAs pending.
    // The wave's own LDS reads complete first, so after the barrier no wave
    // still reads the stage that the next DMA overwrites.
    auto wait_tile = [&](int u) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int ahead = issued - 1 - u;
        if (ahead >= 3) wait_vmcnt<3 * LPT>();
        else if (ahead == 2) wait_vmcnt<2 * LPT>();
        else if (ahead == 1) wait_vmcnt<LPT>();
        else wait_vmcnt<0>();
        barrier_no_fence();
    };
    auto frags = [&](int t, int ks, bf16x8* a, bf16x8* b) {
        const bf16* as = smem + (t % NS) * STAGE;
        const bf16* bs = as + TA::BYTES / 2;
#pragma unroll
        for (int i = 0; i < FM; ++i) a[i] = TA::get(as, wm + 32 * i, ks, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = TB::get(bs, wn + 32 * j, ks, lane);
    };

    for (int t = 0; t < NS; ++t) {
        if (PIPE != PIPE_VGPR && issued < nk) {
            bf16* st = smem + (issued % NS) * STAGE;
#pragma unroll
            for (int q = 0; q < LPT; ++q) dma(q, st);
            ++issued;
        }
    }

    // Software pipeline over 16-deep steps (KS per k-tile):
    //   steps 0 .. KS-2 of tile t: products of step s | reads of step s+1
    //   wait + barrier for tile t+1
    //   DMA of tile t+NS into the stage of tile t (every wave finished
    //   reading tile t before this barrier), issued after the first product;
    //   last step of tile t: products | reads of step 0 of tile t+1
    constexpr int KS = BK / 16;
    static_assert(KS % 2 == 0 && NS <= 4, "even number of 16-deep steps; vmcnt bookkeeping for <= 3 tiles ahead");
    if constexpr (RS) {
        // Register-staged pipeline (KS >= 4), tile t:
        //   step 0: products | reads of steps 1 .. KS-1 of tile t
        //   step 1: after its first product every wave has its fragments of
        //           tile t, so after a barrier the copy of tile t+NS goes into
        //           the stage of tile t
        //   steps 2 .. KS-2: products
        //   wait + barrier for tile t+1
        //   last step: products | reads of step 0 of tile t+1
        static_assert(KS >= 4, "register staging needs four or more steps per k-tile");
        constexpr int NF = FM + FN, P = FM * FN, NR = (KS - 1) * NF;
        bf16x8 ra[KS][FM], rb[KS][FN];
        if (nk > 0) {
            wait_tile(0);
            frags(0, 0, ra[0], rb[0]);
        }
        auto none = [](int) {};
        for (int t = 0; t < nk; ++t) {
            const bf16* as = smem + (t % NS) * STAGE;
            const bf16* bs = as + TA::BYTES / 2;
            auto rd = [&](int p) {
#pragma unroll
                for (int idx = 0; idx < NR; ++idx)
                    if (idx * P / NR == p) {
                        const int s = 1 + idx / NF, f = idx % NF;
                        if (f < FM) ra[s][f] = TA::get(as, wm + 32 * f, s, lane);
                        else rb[s][f - FM] = TB::get(bs, wn + 32 * (f - FM), s, lane);
                    }
            };
            products<FM, FN>(acc, ra[0], rb[0], rd);
            bf16* st = smem + (issued % NS) * STAGE;
            const bool copy = issued < nk;
            // copy q after product slot q * (P * (KS - 2)) / LPT of steps
            // 1 .. KS-2: spread evenly, so that the CU's vector memory unit
            // never receives every wave's copies at once
            auto issue = [&](int slot) {
                if (copy) {
#pragma unroll
                    for (int q = 0; q < LPT; ++q)
                        if (q * P * (KS - 2) / LPT == slot) dma(q, st);
                }
            };
            auto refill = [&](int p) {
                if (p == 0) {
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    barrier_no_fence();
                }
                issue(p);
            };
            products<FM, FN>(acc, ra[1], rb[1], refill);
#pragma unroll
            for (int ks = 2; ks < KS - 1; ++ks)
                products<FM, FN>(acc, ra[ks], rb[ks], [&](int p) { issue((ks - 1) * P + p); });
            if (copy) ++issued;
            if (t + 1 < nk) wait_tile(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            // on the last tile these reads see a stage that holds no new tile; the values are never used
            const bf16* an = smem + ((t + 1) % NS) * STAGE;
            const bf16* bn = an + TA::BYTES / 2;
            auto rd0 = [&](int p) {
                if (p < NF) {
                    const int f = p;
                    if (f < FM) ra[0][f] = TA::get(an, wm + 32 * f, 0, lane);
                    else rb[0][f - FM] = TB::get(bn, wn + 32 * (f - FM), 0, lane);
                }
            };
            products<FM, FN>(acc, ra[KS - 1], rb[KS - 1], rd0);
        }
    } else if constexpr (PIPE == PIPE_F8) {
        // Each v_mfma_f32_32x32x64_f8f6f4 takes 32 bytes of A and of B per lane:
        // the fragments of two consecutive 16-unit steps, in the lower and upper
        // halves of an 8-register operand. A and B put the same k positions in
        // the same lane halves, so the order in which the instruction walks k
        // inside a lane does not change the sum. Tile t (two fp8 steps):
        //   fp8 step 0: products | reads of the second step's fragments
        //   reads done + barrier: every wave is finished with the stage of
        //     tile t, and the copy of tile t+NS goes into it
        //   wait + barrier for tile t+1
        //   fp8 step 1: products | reads of tile t+1's first-step fragments
        static_assert(KS == 4, "two fp8 steps per k-tile");
        constexpr int NF = FM + FN, P = FM * FN;
        i32x8 fa[2][FM], fb[2][FN];
        auto rdf = [&](const bf16* as, const bf16* bs, int j, int idx) {
            const int hh = idx / NF, f = idx % NF, ks = 2 * j + hh;
            if (f < FM) {
                const u32x4 v = __builtin_bit_cast(u32x4, TA::get(as, wm + 32 * f, ks, lane));
                if (hh == 0) fa[j][f].lo = __builtin_bit_cast(s32x4, v);
                else fa[j][f].hi = __builtin_bit_cast(s32x4, v);
            } else {
                const u32x4 v = __builtin_bit_cast(u32x4, TB::get(bs, wn + 32 * (f - FM), ks, lane));
                if (hh == 0) fb[j][f - FM].lo = __builtin_bit_cast(s32x4, v);
                else fb[j][f - FM].hi = __builtin_bit_cast(s32x4, v);
            }
        };
        if (nk > 0) {
            wait_tile(0);
#pragma unroll
            for (int idx = 0; idx < 2 * NF; ++idx) rdf(smem, smem + TA::BYTES / 2, 0, idx);
        }
        for (int t = 0; t < nk; ++t) {
            const bf16* as = smem + (t % NS) * STAGE;
            const bf16* bs = as + TA::BYTES / 2;
            products_f8<FM, FN>(acc, fa[0], fb[0], [&](int p) {
#pragma unroll
                for (int idx = 0; idx < 2 * NF; ++idx)
                    if (idx * P / (2 * NF) == p) rdf(as, bs, 1, idx);
            });
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            barrier_no_fence();
            if (issued < nk) {
                bf16* st = smem + (issued % NS) * STAGE;
#pragma unroll
                for (int q = 0; q < LPT; ++q) dma(q, st);
                ++issued;
            }
            if (t + 1 < nk) wait_tile(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            // on the last tile these reads see a stage that holds no new tile; the values are never used
            const bf16* an = smem + ((t + 1) % NS) * STAGE;
            const bf16* bn = an + TA::BYTES / 2;
            products_f8<FM, FN>(acc, fa[1], fb[1], [&](int p) {
#pragma unroll
                for (int idx = 0; idx < 2 * NF; ++idx)
                    if (idx * P / (2 * NF) == p) rdf(an, bn, 0, idx);
            });
        }
    } else if constexpr (PIPE == PIPE_VGPR) {
        // Tile t (stage t % 2):
        //   step 0 .. : the copy of tile t+1 (in registers since tile t-1) is
        //     written to stage (t+1) % 2, whose tile t-1 every wave finished
        //     reading before the last barrier; after each 16-byte write the
        //     register is reloaded with the same copy of tile t+2
        //   steps 0 .. KS-2: products | reads of the next step
        //   LDS writes done + barrier: tile t+1 is in LDS for every wave
        //   last step: products | reads of step 0 of tile t+1
        static_assert(NS == 2, "two LDS stages");
        constexpr int P = FM * FN;
        static_assert(LPT <= P * (KS - 1), "copies fit in the steps before the barrier");
        // The copies are issued without branches (a branch around them makes
        // the compiler wait for every outstanding load before each LDS
        // write): a load for a k-tile past the last one reads the last
        // k-tile again (the pointers stop advancing there) and its LDS write
        // goes to a stage that is no longer read.
        // Buffer loads: one scalar descriptor per operand and a 32-bit byte
        // offset per copy (the host keeps this mode to operands spanning less
        // than 2 GiB) instead of a 64-bit address per lane and copy.
        u32x4 cp[LPT];
        const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0x7fffffff, 0x00020000);
        const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, 0x7fffffff, 0x00020000);
        int offA[PA], offB[PB];
#pragma unroll
        for (int q = 0; q < PA; ++q) offA[q] = (int)((const char*)srcA[q] - (const char*)A);
#pragma unroll
        for (int q = 0; q < PB; ++q) offB[q] = (int)((const char*)srcB[q] - (const char*)B);
        const int bstA = (int)(2 * stA), bstB = (int)(2 * stB);
        auto gload = [&](int q, bool adv) {
            if (q < PA) {
                cp[q] = __builtin_amdgcn_raw_buffer_load_b128(rA, offA[q], 0, 0);
                offA[q] += adv ? bstA : 0;
            } else {
                cp[q] = __builtin_amdgcn_raw_buffer_load_b128(rB, offB[q - PA], 0, 0);
                offB[q - PA] += adv ? bstB : 0;
            }
        };
        auto swrite = [&](int q, bf16* st) {
            bf16* d = q < PA ? st + (wu * PA + q) * 512 : st + TA::BYTES / 2 + (wu * PB + q - PA) * 512;
            *reinterpret_cast<u32x4*>(d + lane * 8) = cp[q];
        };
        auto lds_ready = [&]() {
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            barrier_no_fence();
        };
        bf16x8 fa[2][FM], fb[2][FN];
        if (nk > 0) {
#pragma unroll
            for (int q = 0; q < LPT; ++q) gload(q, nk > 1);
#pragma unroll
            for (int q = 0; q < LPT; ++q) swrite(q, smem);
#pragma unroll
            for (int q = 0; q < LPT; ++q) gload(q, nk > 2);
            lds_ready();
            frags(0, 0, fa[0], fb[0]);
        }
        for (int t = 0; t < nk; ++t) {
            const bf16* as = smem + (t & 1) * STAGE;
            bf16* st = smem + ((t + 1) & 1) * STAGE;
            const bool adv = t + 3 < nk;
#pragma unroll
            for (int ks = 0; ks < KS - 1; ++ks) {
                // copy q after product slot q * (P * (KS - 1)) / LPT of the tile's
                // first KS - 1 steps: spread evenly, so that the CU's vector
                // memory unit never receives every wave's copies at once
                auto copy = [&](int p) {
#pragma unroll
                    for (int q = 0; q < LPT; ++q)
                        if ((q * P * (KS - 1) / LPT) / P == ks && (q * P * (KS - 1) / LPT) % P == p) {
                            swrite(q, st);
                            gload(q, adv);
                        }
                };
                half_step<FM, FN, TA, TB>(acc, fa[ks & 1], fb[ks & 1], fa[(ks + 1) & 1], fb[(ks + 1) & 1], as,
                                          as + TA::BYTES / 2, wm, wn, ks + 1, lane, copy);
            }
            lds_ready();
            __builtin_amdgcn_sched_barrier(0);
            // on the last tile this prefetch reads a stage that holds no new tile;
            // the values are never used
            auto none = [](int) {};
            half_step<FM, FN, TA, TB>(acc, fa[(KS - 1) & 1], fb[(KS - 1) & 1], fa[0], fb[0], st, st + TA::BYTES / 2,
                                      wm, wn, 0, lane, none);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // LDS writes done before the epilogue reuses the stages
    } else {
    bf16x8 fa[2][FM], fb[2][FN];
    if (nk > 0) {
        wait_tile(0);
        frags(0, 0, fa[0], fb[0]);
    }
    auto none = [](int) {};
    for (int t = 0; t < nk; ++t) {
        {
            const bf16* as = smem + (t % NS) * STAGE;
#pragma unroll
            for (int ks = 0; ks < KS - 1; ++ks)
                half_step<FM, FN, TA, TB>(acc, fa[ks & 1], fb[ks & 1], fa[(ks + 1) & 1], fb[(ks + 1) & 1], as,
                                          as + TA::BYTES / 2, wm, wn, ks + 1, lane, none);
        }
        if (t + 1 < nk) wait_tile(t + 1);
        __builtin_amdgcn_sched_barrier(0);
        {
            // on the last tile this prefetch reads a stage that holds no new tile;
            // the values are never used
            const bf16* as = smem + ((t + 1) % NS) * STAGE;
            bf16* st = smem + (issued % NS) * STAGE;
            const bool copy = issued < nk;
            auto issue = [&](int p) {
#pragma unroll
                for (int q = 0; q < LPT; ++q)
                    if (p == 0 && copy) dma(q, st);
            };
            half_step<FM, FN, TA, TB>(acc, fa[(KS - 1) & 1], fb[(KS - 1) & 1], fa[0], fb[0], as, as + TA::BYTES / 2,
                                      wm, wn, 0, lane, issue);
            if (copy) ++issued;
        }
    }
    }

    // ---- epilogue. Each wave stages one 32-row strip of its sub-tile at a
    // time through LDS (fp32, row-major, row stride WN + 8 so the two row
    // groups of a fragment store fall in different banks), then each lane
    // takes 8 consecutive columns of a row: 16-byte global accesses, with the
    // fused operation applied in fp32 on the way out.
    barrier_no_fence();   // every wave has finished with the k-tile stages
    // CPR 8-column chunks per row, RPI rows per pass of the wave (lanes past
    // RPI * CPR idle when CPR does not divide 64), NIT passes per 32-row strip
    constexpr int SS = WN + 8, CPR = WN / 8, RPI = 64 / CPR, NIT = (32 + RPI - 1) / RPI;
    static_assert(NW * 32 * SS * 4 <= NS * STAGE * 2, "staging strip fits in the stage ring");
    float* stg = reinterpret_cast<float*>(smem_raw) + w * 32 * SS;
    const f32x4* stg4 = reinterpret_cast<const f32x4*>(smem_raw) + w * 8 * SS;
    const int lr = lane & 31, lk = lane >> 5;
    const int cc = lane % CPR, ro = lane / CPR;
    const int col = n0 + wn + 8 * cc;
    const bool cin = col < g.N;              // N % 8 == 0: a chunk is wholly inside or outside
    // column sums of the output (bias gradient), ACT_GRAD only: per lane over
    // its rows, then across the lanes and waves of a column in LDS
    constexpr bool CSUM = !SPLIT && EPI == EPI_ACT_GRAD;
    static_assert(!CSUM || NW * RPI * WN * 4 <= NS * STAGE * 2, "column-sum scratch fits in the stage ring");
    float cs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cs[e] = 0.f;
    float bv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bv[e] = 0.f;
    float osc = 1.f;
    if constexpr (PIPE == PIPE_F8) osc = g.out_scale[0] * g.out_scale[1];
    if constexpr (!SPLIT && (EPI == EPI_BIAS || EPI == EPI_BIAS_ACT || EPI == EPI_BIAS_RESID)) {
        if (cin) {
            const float4 b0 = *reinterpret_cast<const float4*>(g.bias + col);
            const float4 b1 = *reinterpret_cast<const float4*>(g.bias + col + 4);
            bv[0] = b0.x; bv[1] = b0.y; bv[2] = b0.z; bv[3] = b0.w;
            bv[4] = b1.x; bv[5] = b1.y; bv[6] = b1.z; bv[7] = b1.w;
        }
    }
    // epilogues that read global memory (residual, activation derivative,
    // previous gradient) issue a strip's loads before staging it, so their
    // latency overlaps the staging instead of stalling every pass
    constexpr bool PRE = !SPLIT && (EPI == EPI_BIAS_RESID || EPI == EPI_ACT_GRAD || EPI == EPI_ACCUM);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        EpiIn pre[PRE ? NIT : 1];
        if constexpr (PRE) {
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int r = it * RPI + ro;
                const int row = m0 + wm + 32 * i + r;
                const bool act = (32 % RPI == 0 || r < 32) && (64 % CPR == 0 || ro < RPI);
                if (act && row < g.M && cin) pre[it] = epi_load<TC, EPI>(g, row, col);
            }
        }
#pragma unroll
        for (int jf = 0; jf < FN; ++jf)
#pragma unroll
            for (int e = 0; e < 16; ++e) stg[(8 * (e >> 2) + 4 * lk + (e & 3)) * SS + 32 * jf + lr] = acc[i][jf][e];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int r = it * RPI + ro;
            const int row = m0 + wm + 32 * i + r;
            const bool act = (32 % RPI == 0 || r < 32) && (64 % CPR == 0 || ro < RPI);
            if (act && row < g.M && cin) {
                const f32x4 u0 = stg4[r * (SS / 4) + 2 * cc], u1 = stg4[r * (SS / 4) + 2 * cc + 1];
                if constexpr (SPLIT) {
                    float* p = part + ((int64_t)kz * g.M + row) * g.N + col;
                    reinterpret_cast<f32x4*>(p)[0] = u0;
                    reinterpret_cast<f32x4*>(p)[1] = u1;
                } else {
                    float v[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
                    if constexpr (PIPE == PIPE_F8) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] *= osc;
                    }
                    const EpiIn in = PRE ? pre[PRE ? it : 0] : EpiIn{};
                    if constexpr (CSUM) {
                        float y[8];
                        epi_store<TC, EPI, ACT>(g, row, col, v, bv, in, y);
#pragma unroll
                        for (int e = 0; e < 8; ++e) cs[e] += y[e];
                    } else {
                        epi_store<TC, EPI, ACT>(g, row, col, v, bv, in);
                    }
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    if constexpr (CSUM) {
        if (g.cpart) {
            // red[wave][row offset][column of the wave's sub-tile]
            float* red = reinterpret_cast<float*>(smem_raw);
            barrier_no_fence();   // every wave has finished reading its staging strips
            if (64 % CPR == 0 || ro < RPI) {
#pragma unroll
                for (int e = 0; e < 8; ++e) red[(w * RPI + ro) * WN + 8 * cc + e] = cs[e];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            barrier_no_fence();
            for (int c = tid; c < BN; c += NT) {
                const int wc = c / WN, cl = c - wc * WN;   // the column's wave column
                float sum = 0.f;
                for (int wv = wc; wv < NW; wv += WGN)
                    for (int r = 0; r < RPI; ++r) sum += red[(wv * RPI + r) * WN + cl];
                if (n0 + c < g.N) g.cpart[(int64_t)(m0 / BM) * g.N + n0 + c] = sum;
            }
        }
    }
}

// ------------------------------------------------------------------ configurations

// Tile configurations: BM x BN output tile, NS k-tile stages of BK, OCC
// workgroups per CU (register and LDS budget), main-loop form (PIPE) and wave
// grid. Only configurations the dispatcher can choose are instantiated.
enum GemmCfg {
    // LDS-DMA copies of 32-deep k-tiles (any K that is a multiple of 32)
    CFG_256_256 = 0, CFG_128_128, CFG_256_128,
    // LDS-DMA copies of 64-deep k-tiles
    CFG_256_256_K64, CFG_256_192_K64, CFG_128_192_K64, CFG_128_128_K64,
    // register-staged k-tiles
    CFG_128_192_K64R, CFG_128_128_K64R, CFG_256_256_K64R,
    // eight waves, register-staged k-tiles
    CFG_256_256_K64RW8, CFG_256_192_K64RW8,
    // eight waves, copies through registers
    CFG_256_256_K64VW8, CFG_256_192_K64VW8,
    CFG_COUNT
};
static const int cfg_bm[CFG_COUNT] = {256, 128, 256, 256, 256, 128, 128, 128, 128, 256, 256, 256, 256, 256};
static const int cfg_bn[CFG_COUNT] = {256, 128, 128, 256, 192, 192, 128, 192, 128, 256, 256, 192, 256, 192};
static const int cfg_bk[CFG_COUNT] = {32, 32, 32, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64, 64};
static const int cfg_ns[CFG_COUNT] = {4, 4, 3, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2};
static const int cfg_occ[CFG_COUNT] = {1, 2, 2, 1, 1, 2, 2, 2, 2, 1, 1, 1, 1, 1};
static const int cfg_pipe[CFG_COUNT] = {0, 0, 0, 0, 0, 0, 0, 1, 1, 1, 1, 1, 2, 2};
static const int cfg_wgm[CFG_COUNT] = {2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 4, 2, 4};
static const int cfg_wgn[CFG_COUNT] = {2, 2, 2, 2, 2, 2, 2, 2, 2, 2, 4, 2, 4, 2};

// Epilogues with a direct (unsplit) instantiation per operand layout: the
// forward products (both operands k-contiguous) take every epilogue; the
// input gradients (B row-contiguous) store or apply the activation
// derivative; the weight gradients (both row-contiguous) store or accumulate.
// Split-K products run the plain store kernel and apply the epilogue in the
// slice reduction, so they take every epilogue in every layout.
constexpr bool layout_has_epi(bool akc, bool bkc, int epi) {
    return (akc && bkc) || epi == EPI_STORE || (akc && !bkc && epi == EPI_ACT_GRAD) ||
           (!akc && !bkc && epi == EPI_ACCUM);
}

template <int BM, int BN, int BK, int NS, int OCC, int PIPE, int WGM, int WGN, bool AKC, bool BKC, int EPI, int OUTBF,
          int ACT, bool SPLIT>
static void launch(const Gemm& g, dim3 grid, int kps, float* part, hipStream_t s) {
    if constexpr (!SPLIT && !layout_has_epi(AKC, BKC, EPI)) {
        return;   // not instantiated; gemm_mfma_ok sends such products to the portable kernel
    } else {
        constexpr size_t LDS = (size_t)NS * (BM + BN) * BK * sizeof(bf16);
        static_assert(LDS * OCC <= 160 * 1024, "LDS budget");
        auto k = gemm_mfma_kernel<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI, OUTBF, ACT, SPLIT>;
        static bool attr = false;
        if (!attr) {
            (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS);
            attr = true;
        }
        k<<<grid, 64 * WGM * WGN, LDS, s>>>(g, kps, part);
    }
}

// output storage of each epilogue (bf16 except the fp32 residual stream,
// gradient accumulators and fp32 stores)
static int out_bf(const Gemm& g) {
    if (g.epi == EPI_BIAS_RESID || g.epi == EPI_ACCUM) return 0;
    if (g.epi == EPI_STORE) return g.c_bf ? 1 : 0;
    return 1;
}

template <int BM, int BN, int BK, int NS, int OCC, int PIPE, int WGM, int WGN, bool AKC, bool BKC>
static void run_main(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s) {
    dim3 grid(ceil_div(g.N, BN) * ceil_div(g.M, BM), 1, g.batch > 1 ? g.batch : p.splits);
    const int kps = ceil_div(ceil_div(g.K, p.splits), BK) * BK;
    if (p.splits > 1) { launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_STORE, 0, 0, true>(g, grid, kps, part, s); return; }
    const bool relu = g.act == ACT_RELU2;
    switch (g.epi) {
        case EPI_STORE:
            if (g.c_bf) launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_STORE, 1, 0, false>(g, grid, kps, part, s);
            else launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_STORE, 0, 0, false>(g, grid, kps, part, s);
            break;
        case EPI_BIAS: launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_BIAS, 1, 0, false>(g, grid, kps, part, s); break;
        case EPI_BIAS_ACT:
            if (relu) launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_BIAS_ACT, 1, ACT_RELU2, false>(g, grid, kps, part, s);
            else launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_BIAS_ACT, 1, ACT_GELU, false>(g, grid, kps, part, s);
            break;
        case EPI_BIAS_RESID:
            launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_BIAS_RESID, 0, 0, false>(g, grid, kps, part, s);
            break;
        case EPI_ACT_GRAD:
            if (relu) launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_ACT_GRAD, 1, ACT_RELU2, false>(g, grid, kps, part, s);
            else launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_ACT_GRAD, 1, ACT_GELU, false>(g, grid, kps, part, s);
            break;
        case EPI_ACCUM: launch<BM, BN, BK, NS, OCC, PIPE, WGM, WGN, AKC, BKC, EPI_ACCUM, 0, 0, false>(g, grid, kps, part, s); break;
    }
}

template <bool AKC, bool BKC>
static void run_cfg(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s) {
    switch (p.cfg) {
        case CFG_256_256: run_main<256, 256, 32, 4, 1, PIPE_DMA, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_128_128: run_main<128, 128, 32, 4, 2, PIPE_DMA, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_256_128: run_main<256, 128, 32, 3, 2, PIPE_DMA, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_256_256_K64: run_main<256, 256, 64, 2, 1, PIPE_DMA, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_256_192_K64: run_main<256, 192, 64, 2, 1, PIPE_DMA, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_128_192_K64: run_main<128, 192, 64, 2, 2, PIPE_DMA, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_128_128_K64: run_main<128, 128, 64, 2, 2, PIPE_DMA, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_128_192_K64R: run_main<128, 192, 64, 2, 2, PIPE_DMA_RS, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_128_128_K64R: run_main<128, 128, 64, 2, 2, PIPE_DMA_RS, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_256_256_K64R: run_main<256, 256, 64, 2, 1, PIPE_DMA_RS, 2, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_256_256_K64RW8: run_main<256, 256, 64, 2, 1, PIPE_DMA_RS, 2, 4, AKC, BKC>(g, p, part, s); break;
        case CFG_256_192_K64RW8: run_main<256, 192, 64, 2, 1, PIPE_DMA_RS, 4, 2, AKC, BKC>(g, p, part, s); break;
        case CFG_256_256_K64VW8: run_main<256, 256, 64, 2, 1, PIPE_VGPR, 2, 4, AKC, BKC>(g, p, part, s); break;
        case CFG_256_192_K64VW8: run_main<256, 192, 64, 2, 1, PIPE_VGPR, 4, 2, AKC, BKC>(g, p, part, s); break;
    }
}

// One translation unit per operand layout (they compile in parallel):
// kk = X W^T (both k-contiguous), kc = dY W (B row-contiguous),
// cc = dY^T X (both row-contiguous).
void gemm_mfma_run_kk(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s);
void gemm_mfma_run_kc(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s);
void gemm_mfma_run_cc(const Gemm& g, const GemmPlan& p, float* part, hipStream_t s);
// e4m3 product X W^T (both k-contiguous), bf16 store scaled by out_scale[0] * out_scale[1]
void gemm_mfma_run_f8(const Gemm& g, hipStream_t s);

}  // namespace gk
