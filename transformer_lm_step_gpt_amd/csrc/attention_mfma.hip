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
// Streamed 64-row tiles (K, V or Q, dO) are copied into a ring of LDS stages
// by 16-byte LDS-DMA loads and waited for with s_waitcnt vmcnt only when they
// are consumed, so several tiles are in flight. Tiles are kept row-major
// ([row][d], 16-byte chunks swizzled by row); operands that need d as the row
// index are read with the transposing LDS read ds_read_b64_tr_b16.
//
// Accumulator fragments hold rows 8*(e/4) + 4*(lane/32) + e%4 of a 32-row
// block. When such a fragment is reused as the 16-deep k operand of the next
// product, k slot 8*(lane/32) + e' stands for row 8*(e'/4) + 4*(lane/32) +
// e'%4; the other operand is read with the same slot-to-row mapping (two
// transposing reads of 4 consecutive rows), so the product is unchanged.
//
// All outputs are written by exactly one workgroup: no atomics.
#include "common.h"
#include "kernels.h"

namespace gk {

namespace {

constexpr float M_LOG2E_F = 1.4426950408889634f;
constexpr float M_LN2_F = 0.6931471805599453f;
constexpr int ATT_BQ = 128;    // queries (fwd, dQ) or keys (dK dV) per workgroup: 4 waves x 32
constexpr int ATT_BT = 64;     // rows of a streamed tile
constexpr int ATT_NS = 3;      // LDS stages
constexpr int ATT_MAX_T = 4096;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

template <int N>
GPT_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// barrier without the release fence of __syncthreads (which would also wait
// for the LDS-DMA loads still in flight for later tiles)
GPT_DEV void barrier_no_fence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

GPT_DEV f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

GPT_DEV f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.f;
    return z;
}

GPT_DEV bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// evaluated without branches (bitwise and/or of the comparisons)
GPT_DEV bool visible(int q, int key, int T, int W) {
    return (key <= q) & (key < T) & (q < T) & ((W <= 0) | (q - key < W));
}

// A [64][HD] bf16 tile of one head in LDS, filled by LDS-DMA.
template <int HD>
struct HTile {
    static constexpr int CH = HD / 8;               // 16-byte chunks per row
    static constexpr int RPD = 64 / CH;             // rows per wave-wide 1 KiB DMA
    static constexpr int PER_WAVE = ATT_BT / RPD / 4;
    static constexpr int ELEMS = ATT_BT * HD;
    // chunk swizzle by row: 16 consecutive rows read at one chunk (row
    // fragments) and 4 consecutive rows x 4 chunks (transposing reads) both
    // fall in distinct 16-byte bank groups. 8 chunks per row (two rows per
    // 64-bank cycle): the row pair's index with its low bit moved to the top;
    // 16 chunks: the row's two low 2-bit fields swapped.
    GPT_DEV static int swz(int r) {
        if constexpr (CH == 8) {
            const int x = (r >> 1) & 7;
            return ((x & 1) << 2) | (x >> 1);
        } else {
            return ((r & 3) << 2) | ((r >> 2) & 3);
        }
    }
    // element offset of this lane's chunk in the wave's p-th DMA, relative to the tile's first row
    GPT_DEV static uint32_t lane_off(int p, int64_t ld, int w, int lane) {
        const int d = w * PER_WAVE + p;
        const int r = d * RPD + lane / CH;
        const int c = (lane % CH) ^ swz(r);
        return (uint32_t)((int64_t)r * ld + c * 8);
    }
    // a whole tile whose first row is at base, with the lane offsets of lane_off
    GPT_DEV static void load_full(bf16* tile, const bf16* base, const uint32_t (&off)[PER_WAVE], int w) {
#pragma unroll
        for (int p = 0; p < PER_WAVE; ++p) {
            const int d = w * PER_WAVE + p;
            __builtin_amdgcn_global_load_lds(base + off[p], (lds_void_t*)(tile + d * 512), 16, 0, 0);
        }
    }
    // rows r0 .. r0+63 of a [T, *] head slice (row stride ld); rows >= T repeat row T-1
    GPT_DEV static void load(bf16* tile, const bf16* src, int64_t ld, int r0, int T, int w, int lane) {
#pragma unroll
        for (int p = 0; p < PER_WAVE; ++p) {
            const int d = w * PER_WAVE + p;
            const int r = d * RPD + lane / CH;
            const int c = (lane % CH) ^ swz(r);
            const int gr = min(r0 + r, T - 1);
            __builtin_amdgcn_global_load_lds(src + (int64_t)gr * ld + c * 8, (lds_void_t*)(tile + d * 512), 16, 0, 0);
        }
    }
    // 16-deep operand: row r, columns 16*ds + 8*hh .. +8
    GPT_DEV static bf16x8 rowfrag(const bf16* tile, int r, int ds, int hh) {
        const int c = 2 * ds + hh;
        return *reinterpret_cast<const bf16x8*>(tile + r * HD + ((c ^ swz(r)) << 3));
    }
    GPT_DEV static s16x4 tr(const bf16* tile, int r, int d) {
        const bf16* p = tile + r * HD + (((d >> 3) ^ swz(r)) << 3) + (d & 7);
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
    }
    // 16-deep operand with the tile's rows as k: lane l gets column d0 + l%32 and
    // rows 16*ks + 4*(l/32) + {0..3}, then 16*ks + 8 + 4*(l/32) + {0..3}
    GPT_DEV static bf16x8 trfrag(const bf16* tile, int d0, int ks, int lane) {
        const int G = lane >> 4, j = lane & 15;
        const int r = 16 * ks + 4 * (G >> 1) + (j >> 2);
        const int d = d0 + 16 * (G & 1) + 4 * (j & 3);
        s16x4 lo = tr(tile, r, d), hi = tr(tile, r + 8, d);
        u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        u32x4 v = {l2[0], l2[1], h2[0], h2[1]};
        return __builtin_bit_cast(bf16x8, v);
    }
};

// Ring of NS stages, each holding two HTiles (X then Y).
template <int HD, int NS = ATT_NS>
struct TileRing {
    using TL = HTile<HD>;
    static constexpr int STAGE = 2 * TL::ELEMS;
    static constexpr int LPT = 2 * TL::PER_WAVE;    // DMAs per wave per stage
    bf16* smem;
    const bf16 *X, *Y;
    int64_t ldx, ldy;
    int first, ntiles, T, w, lane;
    int issued = 0;
    // per-lane element offsets inside a full tile, kept in registers for head dims
    // <= 64 (the hd-128 kernels have no registers to spare and recompute them)
    static constexpr bool KEEP = HD <= 64;
    uint32_t offx[TL::PER_WAVE], offy[TL::PER_WAVE];
    GPT_DEV void init() {
#pragma unroll
        for (int p = 0; p < TL::PER_WAVE; ++p) {
            offx[p] = KEEP ? TL::lane_off(p, ldx, w, lane) : 0u;
            offy[p] = KEEP ? TL::lane_off(p, ldy, w, lane) : 0u;
        }
    }
    GPT_DEV void issue_next() {
        if (issued < ntiles) {
            bf16* st = smem + (issued % NS) * STAGE;
            const int r0 = first + issued * ATT_BT;
            if (KEEP && r0 + ATT_BT <= T) {
                // whole tile inside the sequence: wave-uniform base plus the lane's offset
                TL::load_full(st, X + (int64_t)r0 * ldx, offx, w);
                TL::load_full(st + TL::ELEMS, Y + (int64_t)r0 * ldy, offy, w);
            } else {
                TL::load(st, X, ldx, r0, T, w, lane);
                TL::load(st + TL::ELEMS, Y, ldy, r0, T, w, lane);
            }
            ++issued;
        }
    }
    // tile u in LDS for every wave; then the stage of tile u-1 is refilled
    GPT_DEV void acquire(int u) {
        if (issued - 1 - u >= 1) wait_vmcnt<LPT>();
        else wait_vmcnt<0>();
        barrier_no_fence();
        issue_next();
    }
    GPT_DEV const bf16* x(int u) const { return smem + (u % NS) * STAGE; }
    GPT_DEV const bf16* y(int u) const { return smem + (u % NS) * STAGE + TL::ELEMS; }
};

// Column sums over the 128 rows of a workgroup (4 waves x 32 lanes) of one
// accumulator set f32x16[NDF] (rows 8*(e/4) + 4*(lane/32) + e%4 of 32-row blocks
// are head dims, lanes are the workgroup's queries or keys), scaled by `scale`,
// lanes with ok = false counting as zero. Summed in LDS in a fixed order (waves,
// then lanes) and written to out[0 .. HD). red: 4 * NDF * 16 * COLSUM_LD floats of LDS
// that no wave reads or writes any more; every thread of the workgroup calls it.
// Rows of red are COLSUM_LD floats apart, so that the reads of the second phase
// (one row per head dim, the same column across the wave) fall in distinct banks.
constexpr int COLSUM_LD = 65;
template <int HD, int NDF>
GPT_DEV void block_colsum(const f32x16 (&acc)[NDF], float scale, bool ok, float* red, float* out, int w, int lane) {
    constexpr int NV = NDF * 16;
    barrier_no_fence();
#pragma unroll
    for (int v = 0; v < NV; ++v) red[(w * NV + v) * COLSUM_LD + lane] = ok ? acc[v / 16][v % 16] * scale : 0.f;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    barrier_no_fence();
    const int d = threadIdx.x;
    if (d < HD) {
        const int df = d >> 5, r = d & 31, half = (r >> 2) & 1, e = ((r >> 3) << 2) | (r & 3);
        const int v = df * 16 + e;
        float sum = 0.f;
        for (int ww = 0; ww < 4; ++ww)
            for (int lr = 0; lr < 32; ++lr) sum += red[(ww * NV + v) * COLSUM_LD + 32 * half + lr];
        out[d] = sum;
    }
}

}  // namespace

// ============================================================== forward

constexpr int ATT_FWD_NS = 2;   // forward: two stages, so four workgroups fit a CU's LDS
template <int HD>
__global__ __launch_bounds__(256, HD == 64 ? 4 : 2) void attn_fwd_mfma_kernel(Attn a) {
    constexpr int NDS = HD / 16, NDF = HD / 32;
    using TL = HTile<HD>;
    constexpr int FNS = ATT_FWD_NS;
    __shared__ __attribute__((aligned(1024))) bf16 smem[FNS * TileRing<HD, FNS>::STAGE];
    // workgroups are dispatched x-fastest: every (batch, head) of the heaviest
    // query tile goes first (longest-first over the whole grid)
    const int qt = gridDim.y - 1 - blockIdx.y;
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const int T = a.T, W = a.window;
    const int q0 = qt * ATT_BQ;
    // the wave index as a wave-uniform (scalar) value, so per-wave tests are scalar branches
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lr = lane & 31,
              hh = lane >> 5;
    const int qw = q0 + w * 32, myq = qw + lr;
    const bf16* Q = (const bf16*)a.q + (int64_t)b * T * a.ldq + h * HD;
    const int kend = min(T, q0 + ATT_BQ);
    int kbeg = W > 0 ? max(0, q0 - W + 1) : 0;
    kbeg = (kbeg / ATT_BT) * ATT_BT;
    TileRing<HD, FNS> ring{smem, (const bf16*)a.k + (int64_t)b * T * a.ldk + h * HD,
                           (const bf16*)a.v + (int64_t)b * T * a.ldv + h * HD, a.ldk, a.ldv, kbeg,
                           ceil_div(kend - kbeg, ATT_BT), T, w, lane};
    ring.init();
    for (int s = 0; s < FNS - 1; ++s) ring.issue_next();

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
    for (int t = 0; t < ring.ntiles; ++t) {
        ring.acquire(t);
        const int kt = kbeg + t * ATT_BT;
        if (kt > qw + 31) continue;                               // the whole tile is in this wave's future
        if (W > 0 && kt + ATT_BT - 1 <= qw - W) continue;          // the whole tile left every window
        const bf16* Ks = ring.x(t);
        const bf16* Vs = ring.y(t);
        f32x16 s[2];
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
            s[kf] = zero16();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s[kf] = mfma(TL::rowfrag(Ks, kf * 32 + lr, ds, hh), qf[ds], s[kf]);
        }
        const bool need_mask = (kt + ATT_BT - 1 > qw) || (kt + ATT_BT > T) || (W > 0 && qw + 31 - kt >= W);
        if (need_mask) {
#pragma unroll
            for (int kf = 0; kf < 2; ++kf)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kt + kf * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                    s[kf][e] = visible(myq, key, T, W) ? s[kf][e] : -INFINITY;
                }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int kf = 0; kf < 2; ++kf)
#pragma unroll
            for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, s[kf][e]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        // The running max is raised only when a score exceeds it by more than
        // 2^8 in exp2 units (and always from -inf): the output and the sum use
        // the same reference, so the result is unchanged while p stays <= 256;
        // the accumulators are rescaled only when some lane of the wave moves.
        if (__builtin_amdgcn_ballot_w64((tmax * c > mrow * c + 8.f) | ((mrow == -INFINITY) & (tmax > -INFINITY)))) {
            const float mnew = fmaxf(mrow, tmax);
            const float mcn = mnew == -INFINITY ? 0.f : mnew * c;
            const float corr = __builtin_amdgcn_exp2f(mrow * c - mcn);
            mrow = mnew;
            lsum *= corr;
#pragma unroll
            for (int df = 0; df < NDF; ++df)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[df][e] *= corr;
        }
        const float mc = mrow == -INFINITY ? 0.f : mrow * c;
        bf16x8 pk[4];
#pragma unroll
        for (int kf = 0; kf < 2; ++kf)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[kf][e], c, -mc));
                lsum += p;
                pk[2 * kf + (e >> 3)][e & 7] = (bf16)p;
            }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int df = 0; df < NDF; ++df) oacc[df] = mfma(TL::trfrag(Vs, df * 32, ks, lane), pk[ks], oacc[df]);
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
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_mfma_kernel(Attn a) {
    constexpr int NDS = HD / 16, NDF = HD / 32;
    using TL = HTile<HD>;
    static_assert(2 * ATT_NS * TileRing<HD>::STAGE >= 4 * NDF * 16 * COLSUM_LD * 4, "column-sum scratch fits in the ring");
    __shared__ __attribute__((aligned(1024))) bf16 smem[ATT_NS * TileRing<HD>::STAGE];
    __shared__ __attribute__((aligned(16))) float Lrow[ATT_MAX_T], Drow[ATT_MAX_T];
    // key blocks in y, (batch, head) in x: the heaviest (first) key blocks of
    // every head are dispatched first
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const int T = a.T, W = a.window;
    const int k0 = blockIdx.y * ATT_BQ;
    // the wave index as a wave-uniform (scalar) value, so per-wave tests are scalar branches
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lr = lane & 31,
              hh = lane >> 5;
    const int kw = k0 + w * 32, mykey = kw + lr;
    const bf16* K = (const bf16*)a.k + (int64_t)b * T * a.ldk + h * HD;
    const bf16* V = (const bf16*)a.v + (int64_t)b * T * a.ldv + h * HD;
    const int qbeg = (k0 / ATT_BT) * ATT_BT;
    const int qend = W > 0 ? min(T, k0 + ATT_BQ - 1 + W) : T;
    TileRing<HD> ring{smem, (const bf16*)a.q + (int64_t)b * T * a.ldq + h * HD,
                      (const bf16*)a.dO + (int64_t)b * T * a.lddo + h * HD, a.ldq, a.lddo, qbeg,
                      ceil_div(qend - qbeg, ATT_BT), T, w, lane};
    ring.init();
    for (int s = 0; s < ATT_NS - 1; ++s) ring.issue_next();

    // log-sum-exp (log2 units) and D = rowsum(dO o O) of every query this workgroup visits
    // (zero past T, so masked positions stay finite)
    for (int i = qbeg + threadIdx.x; i < qbeg + ring.ntiles * ATT_BT; i += 256) {
        Lrow[i - qbeg] = i < T ? a.lse[(int64_t)bh * T + i] * M_LOG2E_F : 0.f;
        Drow[i - qbeg] = i < T ? a.D[(int64_t)bh * T + i] : 0.f;
    }
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
    for (int t = 0; t < ring.ntiles; ++t) {
        ring.acquire(t);   // the barrier also publishes Lrow / Drow on the first tile
        const int qt = qbeg + t * ATT_BT;
        if (qt + ATT_BT - 1 < kw) continue;                         // every query precedes every key of the wave
        if (W > 0 && qt > kw + 31 + W - 1) continue;               // every query is past every window
        const bf16* Qs = ring.x(t);
        const bf16* Gs = ring.y(t);
        const float* Ls = Lrow + (qt - qbeg);
        const float* Ds = Drow + (qt - qbeg);
        const bool need_mask = (qt < kw + 31) || (qt + ATT_BT > T) || (W > 0 && qt + ATT_BT - 1 - kw >= W);
#pragma unroll
        for (int qf = 0; qf < 2; ++qf) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s = mfma(TL::rowfrag(Qs, qf * 32 + lr, ds, hh), kf[ds], s);
                dp = mfma(TL::rowfrag(Gs, qf * 32 + lr, ds, hh), vf[ds], dp);
            }
            float4 lq[4], dq4[4];   // rows 8*g + 4*hh + {0..3} of this q fragment
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                lq[g4] = *reinterpret_cast<const float4*>(Ls + qf * 32 + 8 * g4 + 4 * hh);
                dq4[g4] = *reinterpret_cast<const float4*>(Ds + qf * 32 + 8 * g4 + 4 * hh);
            }
            // P in place of S; the masking is a loop of its own so the unmasked
            // path stays one straight-line block
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c, -(&lq[e >> 2].x)[e & 3]));
            if (need_mask) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int qi = qf * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                    s[e] = visible(qt + qi, mykey, T, W) ? s[e] : 0.f;
                }
            }
            bf16x8 pk[2], dsk[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = s[e], dsv = p * (dp[e] - (&dq4[e >> 2].x)[e & 3]);
                pk[e >> 3][e & 7] = (bf16)p;
                dsk[e >> 3][e & 7] = (bf16)dsv;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int df = 0; df < NDF; ++df) {
                    dv[df] = mfma(TL::trfrag(Gs, df * 32, 2 * qf + kk, lane), pk[kk], dv[df]);
                    dk[df] = mfma(TL::trfrag(Qs, df * 32, 2 * qf + kk, lane), dsk[kk], dk[df]);
                }
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
    if (a.cpart) {   // bias-gradient column sums of this block's dK and dV (values before rounding)
        float* row = a.cpart + (int64_t)(b * gridDim.y + blockIdx.y) * (3 * a.H * HD);
        float* red = reinterpret_cast<float*>(smem);
        block_colsum<HD, NDF>(dk, 1.0f / sqrtf((float)HD), mykey < T, red, row + a.H * HD + h * HD, w, lane);
        block_colsum<HD, NDF>(dv, 1.0f, mykey < T, red, row + 2 * a.H * HD + h * HD, w, lane);
    }
}

// ============================================================== backward: dQ

template <int HD>
__global__ __launch_bounds__(256, HD == 128 ? 2 : 1) void attn_bwd_dq_mfma_kernel(Attn a) {
    constexpr int NDS = HD / 16, NDF = HD / 32;
    using TL = HTile<HD>;
    // hd 128: two stages (64 KiB of tiles, 65 KiB with the column-sum scratch), so
    // two workgroups fit a CU; hd 64: three stages (three workgroups per CU by registers)
    constexpr int DNS = HD == 128 ? 2 : ATT_NS;
    constexpr int RING = DNS * TileRing<HD, DNS>::STAGE, CSUM = 2 * NDF * 16 * COLSUM_LD * 4;   // bf16 elements
    __shared__ __attribute__((aligned(1024))) bf16 smem[RING > CSUM ? RING : CSUM];
    const int qtile = gridDim.y - 1 - blockIdx.y;   // heaviest query tiles of every head first
    const int bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const int T = a.T, W = a.window;
    const int q0 = qtile * ATT_BQ;
    // the wave index as a wave-uniform (scalar) value, so per-wave tests are scalar branches
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lr = lane & 31,
              hh = lane >> 5;
    const int qw = q0 + w * 32, myq = qw + lr;
    const bf16* Q = (const bf16*)a.q + (int64_t)b * T * a.ldq + h * HD;
    const bf16* G = (const bf16*)a.dO + (int64_t)b * T * a.lddo + h * HD;
    const int kend = min(T, q0 + ATT_BQ);
    int kbeg = W > 0 ? max(0, q0 - W + 1) : 0;
    kbeg = (kbeg / ATT_BT) * ATT_BT;
    TileRing<HD, DNS> ring{smem, (const bf16*)a.k + (int64_t)b * T * a.ldk + h * HD,
                      (const bf16*)a.v + (int64_t)b * T * a.ldv + h * HD, a.ldk, a.ldv, kbeg,
                      ceil_div(kend - kbeg, ATT_BT), T, w, lane};
    ring.init();
    for (int s = 0; s < DNS - 1; ++s) ring.issue_next();

    bf16x8 qf[NDS], gf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        bf16x8 z = {};
        qf[ds] = myq < T ? load8(Q + (int64_t)myq * a.ldq + 16 * ds + 8 * hh) : z;
        gf[ds] = myq < T ? load8(G + (int64_t)myq * a.lddo + 16 * ds + 8 * hh) : z;
    }
    const float c = M_LOG2E_F / sqrtf((float)HD);
    const float lse2 = myq < T ? a.lse[(int64_t)bh * T + myq] * M_LOG2E_F : 0.f;
    // D = rowsum(dO o O) of this lane's query: each half-wave holds half of the head dims
    float Dq = 0.f;
    if (myq < T) {
        const bf16* O = (const bf16*)a.o + ((int64_t)b * T + myq) * a.ldo + h * HD;
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            bf16x8 ov = load8(O + 16 * ds + 8 * hh);
#pragma unroll
            for (int e = 0; e < 8; ++e) Dq = fmaf((float)gf[ds][e], (float)ov[e], Dq);
        }
    }
    Dq += __shfl_xor(Dq, 32, 64);
    if (myq < T && hh == 0) a.Dout[(int64_t)bh * T + myq] = Dq;
    f32x16 dq[NDF];
#pragma unroll
    for (int df = 0; df < NDF; ++df) dq[df] = zero16();
    for (int t = 0; t < ring.ntiles; ++t) {
        ring.acquire(t);
        const int kt = kbeg + t * ATT_BT;
        if (kt > qw + 31) continue;
        if (W > 0 && kt + ATT_BT - 1 <= qw - W) continue;
        const bf16* Ks = ring.x(t);
        const bf16* Vs = ring.y(t);
        const bool need_mask = (kt + ATT_BT - 1 > qw) || (kt + ATT_BT > T) || (W > 0 && qw + 31 - kt >= W);
#pragma unroll
        for (int kf = 0; kf < 2; ++kf) {
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s = mfma(TL::rowfrag(Ks, kf * 32 + lr, ds, hh), qf[ds], s);
                dp = mfma(TL::rowfrag(Vs, kf * 32 + lr, ds, hh), gf[ds], dp);
            }
            // P in place of S; the masking is a loop of its own so the unmasked
            // path stays one straight-line block
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = __builtin_amdgcn_exp2f(fmaf(s[e], c, -lse2));
            if (need_mask) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kt + kf * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                    s[e] = visible(myq, key, T, W) ? s[e] : 0.f;
                }
            }
            bf16x8 dsk[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) dsk[e >> 3][e & 7] = (bf16)(s[e] * (dp[e] - Dq));
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int df = 0; df < NDF; ++df)
                    dq[df] = mfma(TL::trfrag(Ks, df * 32, 2 * kf + kk, lane), dsk[kk], dq[df]);
        }
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
    if (a.cpart) {   // bias-gradient column sums of this block's dQ (values before rounding)
        float* row = a.cpart + (int64_t)(b * gridDim.y + qtile) * (3 * a.H * HD);
        block_colsum<HD, NDF>(dq, 1.0f / sqrtf((float)HD), myq < T, reinterpret_cast<float*>(smem), row + h * HD, w,
                              lane);
    }
}

// ============================================================== dispatch

static bool mfma_ok(const Attn& a) {
    if (!a.bf || (a.hd != 64 && a.hd != 128) || a.T > ATT_MAX_T) return false;
    auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (!al(a.q) || !al(a.k) || !al(a.v)) return false;
    if (a.ldq % 8 || a.ldk % 8 || a.ldv % 8) return false;
    return true;
}

bool attention_fwd_mfma(const Attn& a, hipStream_t s) {
    if (!mfma_ok(a) || a.ldo % 4) return false;
    dim3 grid(a.B * a.H, ceil_div(a.T, ATT_BQ));
    if (a.hd == 64) attn_fwd_mfma_kernel<64><<<grid, 256, 0, s>>>(a);
    else attn_fwd_mfma_kernel<128><<<grid, 256, 0, s>>>(a);
    return true;
}

bool attention_bwd_mfma(const Attn& a, hipStream_t s) {
    if (!mfma_ok(a) || a.lddo % 8 || a.ldd % 4 || a.ldo % 8) return false;
    auto al = [](const void* p) { return ((uintptr_t)p & 15) == 0; };
    if (!al(a.dO) || !al(a.o)) return false;
    dim3 grid(a.B * a.H, ceil_div(a.T, ATT_BQ));
    if (a.hd == 64) {
        attn_bwd_dq_mfma_kernel<64><<<grid, 256, 0, s>>>(a);
        attn_bwd_dkdv_mfma_kernel<64><<<grid, 256, 0, s>>>(a);
    } else {
        attn_bwd_dq_mfma_kernel<128><<<grid, 256, 0, s>>>(a);
        attn_bwd_dkdv_mfma_kernel<128><<<grid, 256, 0, s>>>(a);
    }
    return true;
}

}  // namespace gk
