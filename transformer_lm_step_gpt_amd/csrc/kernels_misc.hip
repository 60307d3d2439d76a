// Bandwidth-bound kernels of the GPT-2 training step on gfx950: parameter
// initialisation, embedding forward/backward, LayerNorm forward/backward,
// column sums, fused softmax cross-entropy, attention row dots, q/k
// normalisation + rotary positions, global gradient norm and AdamW.
//
// Model definition: "Zero to Hero, lecture 9: reproducing GPT-2 (124M)"
// (ai.flicky.cc), "Раздел 1 / Архитектура" (pre-LN blocks, final LayerNorm),
// "Генерация и устройство" (token + position embeddings), "Связанные веса и
// инициализация" (tied wte, N(0, 0.02) init with (2 n_layer)^-1/2 on residual
// writers), "Оптимизатор, клиппинг, расписание" (AdamW 0.9/0.95/1e-8, decay
// 0.1 on 2-D tensors, global clip 1.0). Speedrun variants (rotary positions,
// QK-Norm, ReLU^2, softcap): Modded-NanoGPT README (oa0.com), technique list.
#include "common.h"
#include "kernels.h"

#include <mutex>

#include <type_traits>

namespace gk {

// =====================================================================
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) + Box-Muller normals
// =====================================================================

GPT_DEV void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += W0; k1 += W1; }
        uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
        uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
        uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    }
}

__global__ __launch_bounds__(256) void init_normal_kernel(float* dst, int64_t n, uint64_t seed, uint64_t sid,
                                                          double std) {
    int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j * 4 >= n) return;
    uint64_t c[4] = {(uint64_t)j, 0, 0, 0};
    philox4x64_10(c, seed, sid);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        double u1 = ((double)(c[2 * p] >> 11) + 0.5) * 0x1.0p-53;
        double u2 = ((double)(c[2 * p + 1] >> 11) + 0.5) * 0x1.0p-53;
        double r = sqrt(-2.0 * log(u1));
        double t = 6.283185307179586476925 * u2;
        int64_t e = 4 * j + 2 * p;
        if (e < n) dst[e] = (float)(std * (r * cos(t)));
        if (e + 1 < n) dst[e + 1] = (float)(std * (r * sin(t)));
    }
}

void init_normal(float* dst, int64_t n, uint64_t seed, uint64_t sid, double std, hipStream_t s) {
    int64_t blocks = (n + 4 * 256 - 1) / (4 * 256);
    if (blocks) init_normal_kernel<<<(unsigned)blocks, 256, 0, s>>>(dst, n, seed, sid, std);
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* dst, int64_t n, float v) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = v;
}
__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* dst, int64_t n, int32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) dst[i] = v;
}
static unsigned grid_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    return (unsigned)(b < 8192 ? (b < 1 ? 1 : b) : 8192);
}
void fill_f32(float* dst, int64_t n, float v, hipStream_t s) {
    if (n > 0) fill_f32_kernel<<<grid_for(n), 256, 0, s>>>(dst, n, v);
}
void fill_i32(int32_t* dst, int64_t n, int32_t v, hipStream_t s) {
    if (n > 0) fill_i32_kernel<<<grid_for(n), 256, 0, s>>>(dst, n, v);
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(bf16* dst, const float* src, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = (bf16)src[i];
}
void f32_to_bf16(void* dst, const float* src, int64_t n, hipStream_t s) {
    if (n > 0) f32_to_bf16_kernel<<<grid_for(n), 256, 0, s>>>((bf16*)dst, src, n);
}

__global__ void rope_tables_kernel(float* cos_t, float* sin_t, int T, int hd, double base) {
    int half = hd / 2;
    int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * half) return;
    int t = idx / half, i = idx % half;
    double ang = (double)t * pow(base, -2.0 * i / hd);
    cos_t[idx] = (float)cos(ang);
    sin_t[idx] = (float)sin(ang);
}
void rope_tables(float* cos_t, float* sin_t, int T, int hd, double base, hipStream_t s) {
    int n = T * (hd / 2);
    rope_tables_kernel<<<ceil_div(n, 256), 256, 0, s>>>(cos_t, sin_t, T, hd, base);
}

// =====================================================================
// embedding forward: x0 = wte[tok] + wpe[t]
// =====================================================================

__global__ __launch_bounds__(256) void embed_fwd_kernel(const int32_t* tok, const float* wte, const float* wpe,
                                                        float* x0, int M, int T, int d, int Vp, int32_t* err) {
    int dq = d >> 2;
    int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)M * dq) return;
    int m = (int)(idx / dq), c = (int)(idx % dq) * 4;
    int id = tok[m];
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (id >= 0 && id < Vp) {
        v = load4(wte + (int64_t)id * d + c);
    } else if (c == 0) {
        *err = 1;
    }
    if (wpe) {
        float4 p = load4(wpe + (int64_t)(m % T) * d + c);
        v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
    }
    store4(x0 + (int64_t)m * d + c, v);
}

void embed_fwd(const int32_t* tok, const float* wte, const float* wpe, float* x0, int M, int T, int d, int Vp,
               int32_t* err, hipStream_t s) {
    int64_t n = (int64_t)M * (d / 4);
    embed_fwd_kernel<<<ceil_div(n, 256), 256, 0, s>>>(tok, wte, wpe, x0, M, T, d, Vp, err);
}

// =====================================================================
// embedding backward (deterministic, no atomics)
//   1. one workgroup sorts keys (token << 15 | position) with a bitonic
//      network in LDS, then cuts the sorted list into segments (one per
//      distinct token) and pieces (at most PIECE rows of one segment);
//   2. one workgroup per piece sums its rows of dx into a partial row;
//   3. one workgroup per segment adds its pieces' partials, in order, to
//      that token's wte-gradient row.
// =====================================================================

constexpr int EMB_PIECE = 64;
constexpr int EMB_MAXN = 32768;
constexpr int EMB_THREADS = 1024;

struct EmbScratch {
    int32_t* sorted_pos;   // [M]
    int32_t* piece_start;  // [M + 1]
    int32_t* seg_tok;      // [M]
    int32_t* seg_piece;    // [M + 1]
    int32_t* counts;       // [4]: n_valid, n_pieces, n_segs
    float* partial;        // [M, d]
};

static EmbScratch carve_emb(void* base, int M, int d) {
    char* p = (char*)base;
    auto take = [&](size_t bytes) { char* r = p; p += (bytes + 255) & ~size_t(255); return r; };
    EmbScratch e;
    e.sorted_pos = (int32_t*)take(sizeof(int32_t) * M);
    e.piece_start = (int32_t*)take(sizeof(int32_t) * (M + 1));
    e.seg_tok = (int32_t*)take(sizeof(int32_t) * M);
    e.seg_piece = (int32_t*)take(sizeof(int32_t) * (M + 1));
    e.counts = (int32_t*)take(sizeof(int32_t) * 4);
    e.partial = (float*)take(sizeof(float) * (size_t)M * d);
    return e;
}

size_t embed_bwd_scratch_bytes(int M, int d) {
    auto r = [](size_t b) { return (b + 255) & ~size_t(255); };
    return r(4 * (size_t)M) * 2 + r(4 * (size_t)(M + 1)) * 2 + r(16) + r(4 * (size_t)M * d);
}

// Block-wide inclusive scan (sum or max) of one int per thread.
template <bool MAX>
__device__ int block_scan_incl(int v, int* sh /* >= 32 ints */) {
    int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(v, o, 64);
        if (lane >= o) v = MAX ? max(v, u) : v + u;
    }
    if (lane == 63) sh[wid] = v;
    __syncthreads();
    if (wid == 0) {
        int w = lane < nw ? sh[lane] : (MAX ? INT_MIN : 0);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int u = __shfl_up(w, o, 64);
            if (lane >= o) w = MAX ? max(w, u) : w + u;
        }
        if (lane < nw) sh[lane] = w;
    }
    __syncthreads();
    if (wid > 0) { int c = sh[wid - 1]; v = MAX ? max(v, c) : v + c; }
    __syncthreads();
    return v;
}

__global__ __launch_bounds__(EMB_THREADS) void embed_sort_kernel(const int32_t* tok, int M, int Vp, int N,
                                                                  EmbScratch e) {
    extern __shared__ uint32_t keys[];   // N keys
    __shared__ int sh[64];
    const int tid = threadIdx.x;
    for (int i = tid; i < N; i += EMB_THREADS) {
        uint32_t k = 0xFFFFFFFFu;
        if (i < M) {
            int t = tok[i];
            if (t >= 0 && t < Vp) k = ((uint32_t)t << 15) | (uint32_t)i;
        }
        keys[i] = k;
    }
    __syncthreads();
    // bitonic sort, ascending
    for (int size = 2; size <= N; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < N / 2; t += EMB_THREADS) {
                int lo = 2 * t - (t & (stride - 1));
                int hi = lo + stride;
                bool up = (lo & size) == 0;
                uint32_t a = keys[lo], b = keys[hi];
                if ((a > b) == up) { keys[lo] = b; keys[hi] = a; }
            }
            __syncthreads();
        }
    }
    // each thread owns E consecutive sorted entries
    const int E = N / EMB_THREADS;
    const int base = tid * E;
    // pass 1: segment begin (max-scan of segment-start indices)
    int run = INT_MIN;
    for (int u = 0; u < E; ++u) {
        int i = base + u;
        uint32_t k = keys[i];
        bool valid = k != 0xFFFFFFFFu;
        bool start = valid && (i == 0 || (keys[i - 1] >> 15) != (k >> 15));
        if (start) run = i;
    }
    // block_scan_incl folds in every earlier thread; the value this thread
    // starts from is the inclusive result of thread tid - 1
    __shared__ int excl_max[EMB_THREADS];
    int incl = block_scan_incl<true>(run, sh);
    excl_max[tid] = incl;
    __syncthreads();
    int seg_begin = tid ? excl_max[tid - 1] : INT_MIN;
    // pass 2: count pieces and segments owned by this thread
    int npiece = 0, nseg = 0, nvalid = 0;
    {
        int sb = seg_begin;
        for (int u = 0; u < E; ++u) {
            int i = base + u;
            uint32_t k = keys[i];
            bool valid = k != 0xFFFFFFFFu;
            bool start = valid && (i == 0 || (keys[i - 1] >> 15) != (k >> 15));
            if (start) sb = i;
            bool pstart = valid && (start || ((i - sb) % EMB_PIECE) == 0);
            npiece += pstart;
            nseg += start;
            nvalid += valid;
        }
    }
    int pincl = block_scan_incl<false>(npiece, sh);
    int sincl = block_scan_incl<false>(nseg, sh);
    int vincl = block_scan_incl<false>(nvalid, sh);
    int pid = pincl - npiece, sid = sincl - nseg;
    {
        int sb = seg_begin;
        for (int u = 0; u < E; ++u) {
            int i = base + u;
            uint32_t k = keys[i];
            bool valid = k != 0xFFFFFFFFu;
            if (!valid) continue;
            bool start = (i == 0 || (keys[i - 1] >> 15) != (k >> 15));
            if (start) sb = i;
            bool pstart = start || ((i - sb) % EMB_PIECE) == 0;
            e.sorted_pos[i] = (int32_t)(k & 0x7FFF);
            if (start) {
                e.seg_tok[sid] = (int32_t)(k >> 15);
                e.seg_piece[sid] = pid;
                ++sid;
            }
            if (pstart) {
                e.piece_start[pid] = i;
                ++pid;
            }
        }
    }
    if (tid == EMB_THREADS - 1) {
        e.counts[0] = vincl;
        e.counts[1] = pincl;
        e.counts[2] = sincl;
        e.piece_start[pincl] = vincl;
        e.seg_piece[sincl] = pincl;
    }
}

// acc += rows src(0) .. src(n-1), added one by one in that order, with the
// loads of EMB_AHEAD rows in flight at a time (a row's address comes from
// the sorted order, so a plain loop would wait for every row in turn)
constexpr int EMB_AHEAD = 8;
template <typename F>
GPT_DEV float4 emb_sum_rows(float4 acc, int n, F src) {
    int r = 0;
    for (; r + EMB_AHEAD <= n; r += EMB_AHEAD) {
        float4 v[EMB_AHEAD];
#pragma unroll
        for (int u = 0; u < EMB_AHEAD; ++u) v[u] = load4(src(r + u));
#pragma unroll
        for (int u = 0; u < EMB_AHEAD; ++u) {
            acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
        }
    }
    for (; r < n; ++r) {
        const float4 v = load4(src(r));
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    return acc;
}

__global__ __launch_bounds__(256) void embed_piece_kernel(const float* dx, int d, EmbScratch e) {
    int p = blockIdx.x;
    if (p >= e.counts[1]) return;
    int r0 = e.piece_start[p], r1 = e.piece_start[p + 1];
    for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
        const float4 acc = emb_sum_rows(make_float4(0.f, 0.f, 0.f, 0.f), r1 - r0,
                                        [&](int r) { return dx + (int64_t)e.sorted_pos[r0 + r] * d + c; });
        store4(e.partial + (int64_t)p * d + c, acc);
    }
}

__global__ __launch_bounds__(256) void embed_segment_kernel(float* dwte, int d, EmbScratch e) {
    int sidx = blockIdx.x;
    if (sidx >= e.counts[2]) return;
    int p0 = e.seg_piece[sidx], p1 = e.seg_piece[sidx + 1];
    int64_t row = e.seg_tok[sidx];
    for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
        const float4 acc = emb_sum_rows(load4(dwte + row * d + c), p1 - p0,
                                        [&](int q) { return e.partial + (int64_t)(p0 + q) * d + c; });
        store4(dwte + row * d + c, acc);
    }
}

// dwpe[t] (+)= sum over b of dx[b, t] (the previous value dropped when overwrite)
__global__ __launch_bounds__(256) void embed_wpe_kernel(const float* dx, float* dwpe, int B, int T, int d,
                                                        int overwrite) {
    int dq = d >> 2;
    int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * dq) return;
    int t = idx / dq, c = (idx % dq) * 4;
    const float4 acc = emb_sum_rows(overwrite ? make_float4(0.f, 0.f, 0.f, 0.f) : load4(dwpe + (int64_t)t * d + c), B,
                                    [&](int b) { return dx + ((int64_t)b * T + t) * d + c; });
    store4(dwpe + (int64_t)t * d + c, acc);
}

void embed_bwd_sort(const int32_t* tok, int B, int T, int d, int Vp, void* scratch, hipStream_t s) {
    int M = B * T;
    int N = EMB_THREADS;
    while (N < M) N <<= 1;
    EmbScratch e = carve_emb(scratch, M, d);
    size_t lds = sizeof(uint32_t) * (size_t)N;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)embed_sort_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(sizeof(uint32_t) * EMB_MAXN));
        attr_set = true;
    }
    embed_sort_kernel<<<1, EMB_THREADS, lds, s>>>(tok, M, Vp, N, e);
}

void embed_bwd_accumulate(const float* dx, float* dwte, float* dwpe, int B, int T, int d, void* scratch,
                          hipStream_t s, bool overwrite_wpe) {
    const int M = B * T;
    EmbScratch e = carve_emb(scratch, M, d);
    embed_piece_kernel<<<M, 256, 0, s>>>(dx, d, e);
    embed_segment_kernel<<<M, 256, 0, s>>>(dwte, d, e);
    if (dwpe)
        embed_wpe_kernel<<<ceil_div((int64_t)T * (d / 4), 256), 256, 0, s>>>(dx, dwpe, B, T, d, overwrite_wpe ? 1 : 0);
}

void embed_bwd(const int32_t* tok, const float* dx, float* dwte, float* dwpe, int B, int T, int d, int Vp,
               void* scratch, hipStream_t s) {
    embed_bwd_sort(tok, B, T, d, Vp, scratch, s);
    embed_bwd_accumulate(dx, dwte, dwpe, B, T, d, scratch, s);
}

// =====================================================================
// LayerNorm (one wavefront per row; d <= 2048)
// =====================================================================

constexpr int LN_MAXV = 8;   // float4 chunks per lane: d <= 64 * 4 * 8

constexpr int LNF_ROWS = 1;   // rows per wavefront in the forward pass

// One wavefront per LNF_ROWS consecutive rows, all of them loaded before the
// first row's reductions; the gains and biases are loaded once per wave.
// (One row per wave with hoisted gains: 13.1 us for 16384 x 768 alone, 72% of
// HBM peak; four rows per wave with per-row gain loads took 16.7 us.)
template <typename TO, int NV>
__global__ __launch_bounds__(256) void layernorm_fwd_kernel(const float* __restrict__ x, const float* __restrict__ g,
                                                            const float* __restrict__ b, TO* __restrict__ y,
                                                            float* __restrict__ mean, float* __restrict__ rstd, int M,
                                                            int d, float eps) {
    const int lane = threadIdx.x & 63;
    const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * LNF_ROWS, r1 = min(M, r0 + LNF_ROWS);
    const int nv = d >> 2;
    // every row of the wave is loaded before the first is reduced: one memory
    // latency per wave instead of one per row
    float4 rows[LNF_ROWS][NV];
#pragma unroll
    for (int k = 0; k < LNF_ROWS; ++k) {
        const float* xr = x + (int64_t)(r0 + k) * d;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = lane + 64 * i;
            rows[k][i] = (r0 + k < r1 && c < nv) ? load4(xr + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    float4 gg[NV], bb[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        gg[i] = c < nv ? load4(g + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
        bb[i] = c < nv ? load4(b + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int k = 0; k < LNF_ROWS; ++k) {
        const int row = r0 + k;
        if (row >= r1) break;
        const float4 (&cur)[NV] = rows[k];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) s += (cur[i].x + cur[i].y) + (cur[i].z + cur[i].w);
        const float mu = wave_sum(s) / d;
        float s2 = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = lane + 64 * i;
            if (c < nv) {
                const float a = cur[i].x - mu, bb = cur[i].y - mu, cc = cur[i].z - mu, dd = cur[i].w - mu;
                s2 += (a * a + bb * bb) + (cc * cc + dd * dd);
            }
        }
        const float var = wave_sum(s2) / d;
        const float rs = 1.0f / sqrtf(var + eps);
        TO* yr = y + (int64_t)row * d;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int c = lane + 64 * i;
            if (c < nv) {
                float4 o;
                o.x = (cur[i].x - mu) * rs * gg[i].x + bb[i].x;
                o.y = (cur[i].y - mu) * rs * gg[i].y + bb[i].y;
                o.z = (cur[i].z - mu) * rs * gg[i].z + bb[i].z;
                o.w = (cur[i].w - mu) * rs * gg[i].w + bb[i].w;
                store4(yr + 4 * c, o);
            }
        }
        if (lane == 0) { mean[row] = mu; rstd[row] = rs; }
    }
}

template <typename TO>
static void lnf_launch(int nv, int grid, const float* x, const float* g, const float* b, TO* y, float* mean,
                       float* rstd, int M, int d, float eps, hipStream_t s) {
    switch (nv) {
        case 1: layernorm_fwd_kernel<TO, 1><<<grid, 256, 0, s>>>(x, g, b, y, mean, rstd, M, d, eps); break;
        case 2: layernorm_fwd_kernel<TO, 2><<<grid, 256, 0, s>>>(x, g, b, y, mean, rstd, M, d, eps); break;
        case 3: layernorm_fwd_kernel<TO, 3><<<grid, 256, 0, s>>>(x, g, b, y, mean, rstd, M, d, eps); break;
        case 4: layernorm_fwd_kernel<TO, 4><<<grid, 256, 0, s>>>(x, g, b, y, mean, rstd, M, d, eps); break;
        default: layernorm_fwd_kernel<TO, 8><<<grid, 256, 0, s>>>(x, g, b, y, mean, rstd, M, d, eps); break;
    }
}

void layernorm_fwd(bool bf, const float* x, const float* g, const float* b, void* y, float* mean, float* rstd,
                   int M, int d, float eps, hipStream_t s) {
    const int grid = ceil_div(M, 4 * LNF_ROWS), nv = ceil_div(d, 256);
    if (bf) lnf_launch<bf16>(nv, grid, x, g, b, (bf16*)y, mean, rstd, M, d, eps, s);
    else lnf_launch<float>(nv, grid, x, g, b, (float*)y, mean, rstd, M, d, eps, s);
}

constexpr int LNB_ROWS = 32;   // rows per workgroup in the backward pass (8 per wavefront)

// partial sums: [3][nb][d] (dgamma, dbeta, column sums of the new dres) + reduction scratch
size_t layernorm_bwd_partial_floats(int M, int d) {
    int nb = ceil_div(M, LNB_ROWS);
    return (size_t)3 * nb * d + (size_t)3 * ceil_div(nb, 64) * d;
}

// dy as loaded: 4 fp32, or 4 bf16 kept packed until the row is processed
template <typename TD> struct LnbDy { using T = float4; };
template <> struct LnbDy<bf16> { using T = uint2; };
GPT_DEV float4 lnb_dy_load(const float* p) { return load4(p); }
GPT_DEV uint2 lnb_dy_load(const bf16* p) { return *reinterpret_cast<const uint2*>(p); }
GPT_DEV float4 lnb_dy_f(const float4& v) { return v; }
GPT_DEV float4 lnb_dy_f(const uint2& v) {
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                       __uint_as_float(v.y & 0xffff0000u));
}

// one row's inputs in registers: x, dy and the previous residual gradient
template <typename TD, int NV>
struct LnbIn {
    float4 x[NV], old[NV];
    typename LnbDy<TD>::T dy[NV];
    float mu, rs;
};

template <typename TD, int NV>
GPT_DEV void lnb_load(LnbIn<TD, NV>& in, const TD* __restrict__ dy, const float* __restrict__ x,
                      const float* __restrict__ dres, float mu, float rs, int overwrite, int lane, int d) {
    in.mu = mu;
    in.rs = rs;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
        const bool in_row = 4 * c < d;
        in.x[i] = in_row ? load4(x + 4 * c) : z;
        in.dy[i] = in_row ? lnb_dy_load(dy + 4 * c) : typename LnbDy<TD>::T{};
        in.old[i] = (in_row && !overwrite) ? load4(dres + 4 * c) : z;
    }
}

// One row: dx = rstd (dh - mean(dh) - xhat mean(dh xhat)), dh = dy * gamma,
// added to the previous residual gradient; acc(q, i, a, b) adds a * b to the
// lane's column sums q of dy * xhat (dgamma), dy (dbeta) and the new residual
// gradient (b = 1 for the last two)
template <typename TL, typename TD, int NV, typename ACC>
GPT_DEV void lnb_row(const LnbIn<TD, NV>& in, const float4* gg, float* __restrict__ dres, TL* __restrict__ dres_lp,
                     int lane, int d, ACC&& acc) {
    const float mu = in.mu, rs = in.rs;
    float4 xh[NV], dh[NV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const float4 xv = in.x[i], dyv = lnb_dy_f(in.dy[i]);
        xh[i] = make_float4((xv.x - mu) * rs, (xv.y - mu) * rs, (xv.z - mu) * rs, (xv.w - mu) * rs);
        dh[i] = make_float4(dyv.x * gg[i].x, dyv.y * gg[i].y, dyv.z * gg[i].z, dyv.w * gg[i].w);
        s1 += (dh[i].x + dh[i].y) + (dh[i].z + dh[i].w);
        s2 += (dh[i].x * xh[i].x + dh[i].y * xh[i].y) + (dh[i].z * xh[i].z + dh[i].w * xh[i].w);
    }
    s1 = wave_sum(s1) / d;
    s2 = wave_sum(s2) / d;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        if (4 * c < d) {
            const float4 old = in.old[i], dyv = lnb_dy_f(in.dy[i]);
            float4 o;
            o.x = old.x + rs * (dh[i].x - s1 - xh[i].x * s2);
            o.y = old.y + rs * (dh[i].y - s1 - xh[i].y * s2);
            o.z = old.z + rs * (dh[i].z - s1 - xh[i].z * s2);
            o.w = old.w + rs * (dh[i].w - s1 - xh[i].w * s2);
            store4(dres + 4 * c, o);
            if (dres_lp) store4(dres_lp + 4 * c, o);
            acc(0, i, dyv, xh[i]);
            acc(1, i, dyv, make_float4(1.f, 1.f, 1.f, 1.f));
            acc(2, i, o, make_float4(1.f, 1.f, 1.f, 1.f));
        }
    }
}

// Rows are processed with the next row's loads in flight (two row buffers).
// dy (the gradient at the LayerNorm output) is fp32 or bf16 (TD), kept packed
// until its row is processed. Up to d = 1024 each wave keeps its three column
// sums in its own LDS rows (lane-private slots: 36 KiB per workgroup at
// d = 768), so the registers hold only the row buffers and, up to d = 768,
// three workgroups fit a CU; wider rows keep the sums in registers and stage
// one set at a time for the workgroup's sum.
template <int NV>
constexpr bool lnb_acc_lds() { return NV <= 4; }
template <typename TL, typename TD, int NV>
__global__ __launch_bounds__(256, NV <= 3 ? 3 : 2) void layernorm_bwd_kernel(
    const TD* __restrict__ dy, const float* __restrict__ x, const float* __restrict__ mean,
    const float* __restrict__ rstd, const float* __restrict__ g, float* __restrict__ dres, TL* __restrict__ dres_lp,
    int overwrite, float* __restrict__ part, int M, int d) {
    constexpr bool ACC_LDS = lnb_acc_lds<NV>();
    constexpr int DW = 256 * NV, NSET = ACC_LDS ? 3 : 1;
    __shared__ __attribute__((aligned(16))) float red[4][NSET][DW];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nb = gridDim.x;
    float4 gg[NV];
    float4 racc[ACC_LDS ? 1 : 3][NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = lane + 64 * i;
        gg[i] = 4 * c < d ? load4(g + 4 * c) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            if constexpr (ACC_LDS) *reinterpret_cast<float4*>(&red[w][ACC_LDS ? q : 0][4 * c]) = make_float4(0.f, 0.f, 0.f, 0.f);
            else racc[ACC_LDS ? 0 : q][i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    auto acc = [&](int q, int i, float4 a, float4 b) {
        float4* p = ACC_LDS ? reinterpret_cast<float4*>(&red[w][ACC_LDS ? q : 0][4 * (lane + 64 * i)])
                            : &racc[ACC_LDS ? 0 : q][i];
        float4 v = *p;
        v.x = fmaf(a.x, b.x, v.x); v.y = fmaf(a.y, b.y, v.y); v.z = fmaf(a.z, b.z, v.z); v.w = fmaf(a.w, b.w, v.w);
        *p = v;
    };
    constexpr int RPW = LNB_ROWS / 4;   // rows per wave
    const int r0 = blockIdx.x * LNB_ROWS + w * RPW;
    const int r1 = min(M, r0 + RPW);
    auto load_row = [&](LnbIn<TD, NV>& in, int r) {
        const int64_t o = (int64_t)r * d;
        lnb_load<TD, NV>(in, dy + o, x + o, dres + o, mean[r], rstd[r], overwrite, lane, d);
    };
    auto do_row = [&](const LnbIn<TD, NV>& in, int r) {
        const int64_t o = (int64_t)r * d;
        lnb_row<TL, TD, NV>(in, gg, dres + o, dres_lp ? dres_lp + o : nullptr, lane, d, acc);
    };
    LnbIn<TD, NV> b0, b1;
    if (r0 < r1) load_row(b0, r0);
#pragma unroll 1
    for (int k = 0; k < RPW; k += 2) {
        if (r0 + k + 1 < r1) load_row(b1, r0 + k + 1);
        if (r0 + k < r1) do_row(b0, r0 + k);
        if (r0 + k + 2 < r1) load_row(b0, r0 + k + 2);
        if (r0 + k + 1 < r1) do_row(b1, r0 + k + 1);
    }
    // the workgroup's partial sums, its waves added in a fixed order
#pragma unroll
    for (int q = 0; q < 3; ++q) {
        if constexpr (!ACC_LDS) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int c = lane + 64 * i;
                if (4 * c < d) *reinterpret_cast<float4*>(&red[w][0][4 * c]) = racc[ACC_LDS ? 0 : q][i];
            }
        }
        if (!ACC_LDS || q == 0) __syncthreads();
        const int sq = ACC_LDS ? q : 0;
        for (int c = threadIdx.x; c < d; c += 256)
            part[((int64_t)q * nb + blockIdx.x) * d + c] = ((red[0][sq][c] + red[1][sq][c]) + red[2][sq][c]) + red[3][sq][c];
        if (!ACC_LDS) __syncthreads();
    }
}

// out[q][c] += sum_p part[q][p][c] for q < nq, in two deterministic passes
// (groups of 64 partials, then the group sums); tmp holds nq * ceil(np/64) * n floats
__global__ __launch_bounds__(256) void reduce_partials_stage1(const float* part, int np, int n, float* tmp) {
    const int c = blockIdx.x * 256 + threadIdx.x, grp = blockIdx.y, q = blockIdx.z;
    if (c >= n) return;
    const int ng = gridDim.y;
    const int p0 = grp * 64, p1 = min(np, p0 + 64);
    const float* src = part + (int64_t)q * np * n + c;
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    int p = p0;
    for (; p + 4 <= p1; p += 4) {
        a0 += src[(int64_t)p * n];
        a1 += src[(int64_t)(p + 1) * n];
        a2 += src[(int64_t)(p + 2) * n];
        a3 += src[(int64_t)(p + 3) * n];
    }
    for (; p < p1; ++p) a0 += src[(int64_t)p * n];
    tmp[((int64_t)q * ng + grp) * n + c] = (a0 + a1) + (a2 + a3);
}
__global__ __launch_bounds__(256) void reduce_partials_stage2(const float* tmp, int ng, int n, float* out0,
                                                              float* out1, float* out2) {
    const int c = blockIdx.x * 256 + threadIdx.x, q = blockIdx.y;
    if (c >= n) return;
    float* out = q == 0 ? out0 : (q == 1 ? out1 : out2);
    if (!out) return;
    float a = 0.f;
    for (int g = 0; g < ng; ++g) a += tmp[((int64_t)q * ng + g) * n + c];
    out[c] += a;
}

static void reduce_partials(const float* part, int np, int n, int nq, float* tmp, float* o0, float* o1, float* o2,
                            hipStream_t s) {
    const int ng = ceil_div(np, 64);
    reduce_partials_stage1<<<dim3(ceil_div(n, 256), ng, nq), 256, 0, s>>>(part, np, n, tmp);
    reduce_partials_stage2<<<dim3(ceil_div(n, 256), nq), 256, 0, s>>>(tmp, ng, n, o0, o1, o2);
}

// ---- deferred reductions: every job in one pair of launches
size_t reduce_jobs_tmp_floats(int njobs, int max_np, int max_n) {
    return (size_t)njobs * ceil_div(max_np, 64) * max_n;
}

// tmp[job][grp][c] = sum of partial rows 64 grp .. 64 grp + 63 of the job
__global__ __launch_bounds__(256) void reduce_jobs_stage1(const RedJob* __restrict__ jobs, int G, int max_n,
                                                          float* __restrict__ tmp) {
    const RedJob jb = jobs[blockIdx.z];
    const int c = blockIdx.x * 256 + threadIdx.x, grp = blockIdx.y;
    const int p0 = grp * 64, p1 = min(jb.np, p0 + 64);
    if (c >= jb.n || p0 >= p1) return;
    const float* src = jb.part + c;
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = 0.f;
    int p = p0;
    // 32 rows loaded together, added in the same order as eight at a time
    for (; p + 32 <= p1; p += 32) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = src[(int64_t)(p + j) * jb.n];
#pragma unroll
        for (int j = 0; j < 32; ++j) a[j & 7] += v[j];
    }
    for (; p + 8 <= p1; p += 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] += src[(int64_t)(p + e) * jb.n];
    }
    for (; p < p1; ++p) a[0] += src[(int64_t)p * jb.n];
    tmp[((int64_t)blockIdx.z * G + grp) * max_n + c] = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// out[c] += sum of the job's group sums, in group order
__global__ __launch_bounds__(256) void reduce_jobs_stage2(const RedJob* __restrict__ jobs, int G, int max_n,
                                                          const float* __restrict__ tmp, int overwrite) {
    const RedJob jb = jobs[blockIdx.y];
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= jb.n) return;
    const int ng = ceil_div(jb.np, 64);
    float a = 0.f;
    for (int grp = 0; grp < ng; ++grp) a += tmp[((int64_t)blockIdx.y * G + grp) * max_n + c];
    if (overwrite) jb.out[c] = a;
    else jb.out[c] += a;
}

void reduce_jobs(const RedJob* jobs, int njobs, int max_np, int max_n, float* tmp, hipStream_t s, bool overwrite) {
    if (njobs <= 0) return;
    const int G = ceil_div(max_np, 64);
    reduce_jobs_stage1<<<dim3(ceil_div(max_n, 256), G, njobs), 256, 0, s>>>(jobs, G, max_n, tmp);
    reduce_jobs_stage2<<<dim3(ceil_div(max_n, 256), njobs), 256, 0, s>>>(jobs, G, max_n, tmp, overwrite ? 1 : 0);
}

void reduce_rows(const float* part, int np, int n, float* out, float* tmp, hipStream_t s) {
    reduce_partials(part, np, n, 1, tmp, out, nullptr, nullptr, s);
}

template <typename TL, typename TD>
static void lnb_launch(int nv, int nb, const TD* dy, const float* x, const float* mean, const float* rstd,
                       const float* g, float* dres, TL* lp, int ov, float* part, int M, int d, hipStream_t s) {
    switch (nv) {
        case 1: layernorm_bwd_kernel<TL, TD, 1><<<nb, 256, 0, s>>>(dy, x, mean, rstd, g, dres, lp, ov, part, M, d); break;
        case 2: layernorm_bwd_kernel<TL, TD, 2><<<nb, 256, 0, s>>>(dy, x, mean, rstd, g, dres, lp, ov, part, M, d); break;
        case 3: layernorm_bwd_kernel<TL, TD, 3><<<nb, 256, 0, s>>>(dy, x, mean, rstd, g, dres, lp, ov, part, M, d); break;
        case 4: layernorm_bwd_kernel<TL, TD, 4><<<nb, 256, 0, s>>>(dy, x, mean, rstd, g, dres, lp, ov, part, M, d); break;
        default: layernorm_bwd_kernel<TL, TD, 8><<<nb, 256, 0, s>>>(dy, x, mean, rstd, g, dres, lp, ov, part, M, d); break;
    }
}

int layernorm_bwd_num_partials(int M) { return ceil_div(M, LNB_ROWS); }

void layernorm_bwd_rows(bool bf, const void* dy, bool dy_bf, const float* x, const float* mean, const float* rstd,
                        const float* g, float* dres, void* dres_lp, bool overwrite, float* partial, int M, int d,
                        hipStream_t s) {
    const int nb = ceil_div(M, LNB_ROWS);
    const int nv = ceil_div(d, 256);
    if (bf && dy_bf)
        lnb_launch<bf16, bf16>(nv, nb, (const bf16*)dy, x, mean, rstd, g, dres, (bf16*)dres_lp, overwrite, partial, M, d, s);
    else if (bf)
        lnb_launch<bf16, float>(nv, nb, (const float*)dy, x, mean, rstd, g, dres, (bf16*)dres_lp, overwrite, partial, M, d,
                                s);
    else
        lnb_launch<float, float>(nv, nb, (const float*)dy, x, mean, rstd, g, dres, (float*)dres_lp, overwrite, partial, M,
                                 d, s);
}

void layernorm_bwd(bool bf, const float* dy, const float* x, const float* mean, const float* rstd, const float* g,
                   float* dres, void* dres_lp, bool overwrite, float* dg, float* db, float* dcol, float* partial,
                   int M, int d, hipStream_t s) {
    const int nb = ceil_div(M, LNB_ROWS);
    layernorm_bwd_rows(bf, dy, false, x, mean, rstd, g, dres, dres_lp, overwrite, partial, M, d, s);
    reduce_partials(partial, nb, d, dcol ? 3 : 2, partial + (size_t)3 * nb * d, dg, db, dcol, s);
}

// ---- LayerNorm backward without a caller-provided workspace
// The row pass's partial sums and the reduction's group sums live in this
// file-scope device array: one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in symbol); it looks up each device's address once with
// hipGetSymbolAddress and passes that. Every element the kernels read is
// written earlier in the same call, so nothing needs clearing; calls that
// overlap on one GPU share the array and race.
constexpr size_t LNB_STATIC_FLOATS = (size_t)8 << 20;   // 32 MiB
static __device__ __align__(256) float ln_bwd_scratch[LNB_STATIC_FLOATS];
constexpr int LNB_STATIC_MAX_DEVICES = 64;

size_t layernorm_bwd_static_capacity_floats() { return LNB_STATIC_FLOATS; }

int layernorm_bwd_static(bool bf, const float* dy, const float* x, const float* mean, const float* rstd,
                         const float* g, float* dres, void* dres_lp, bool overwrite, float* dg, float* db,
                         float* dcol, int M, int d, hipStream_t s) {
    if (layernorm_bwd_partial_floats(M, d) > LNB_STATIC_FLOATS) return -1;
    static std::mutex mu;
    static float* addr[LNB_STATIC_MAX_DEVICES] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= LNB_STATIC_MAX_DEVICES) return -4;
    float* part = nullptr;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (!addr[dev]) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(ln_bwd_scratch)) != hipSuccess || !p) return -4;
            addr[dev] = (float*)p;
        }
        part = addr[dev];
    }
    layernorm_bwd(bf, dy, x, mean, rstd, g, dres, dres_lp, overwrite, dg, db, dcol, part, M, d, s);
    return 0;
}

// =====================================================================
// column sums (bias gradients): 8 columns per thread, 64 rows per workgroup
// =====================================================================

constexpr int CS_ROWS = 64;

template <typename TI>
__global__ __launch_bounds__(256) void colsum_scalar_kernel(const TI* Y, int64_t ld, int M, int N, float* part) {
    int n = blockIdx.x * 256 + threadIdx.x;
    if (n >= N) return;
    int r0 = blockIdx.y * CS_ROWS, r1 = min(M, r0 + CS_ROWS);
    float a = 0.f;
    for (int r = r0; r < r1; ++r) a += to_f32(Y[(int64_t)r * ld + n]);
    part[(int64_t)blockIdx.y * N + n] = a;
}
size_t colsum_partial_floats(int M, int N) {
    int np = ceil_div(M, CS_ROWS);
    return (size_t)np * N + (size_t)ceil_div(np, 64) * N;
}

// one wavefront per (512-column strip, CS_ROWS-row block): lane = 8 columns,
// 8 rows' 16-byte loads in flight per lane
template <typename TI>
__global__ __launch_bounds__(64) void colsum_kernel(const TI* __restrict__ Y, int64_t ld, int M, int N,
                                                   float* __restrict__ part) {
    const int c0 = (blockIdx.x * 64 + threadIdx.x) * 8;
    if (c0 >= N) return;
    const int r0 = blockIdx.y * CS_ROWS, r1 = min(M, r0 + CS_ROWS);
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = 0.f;
    if (c0 + 8 <= N) {
        int r = r0;
        for (; r + 8 <= r1; r += 8) {
            float4 u[8], v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const TI* p = Y + (int64_t)(r + i) * ld + c0;
                u[i] = load4(p);
                v[i] = load4(p + 4);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a[0] += u[i].x; a[1] += u[i].y; a[2] += u[i].z; a[3] += u[i].w;
                a[4] += v[i].x; a[5] += v[i].y; a[6] += v[i].z; a[7] += v[i].w;
            }
        }
        for (; r < r1; ++r) {
            const TI* p = Y + (int64_t)r * ld + c0;
            const float4 u = load4(p), v = load4(p + 4);
            a[0] += u.x; a[1] += u.y; a[2] += u.z; a[3] += u.w;
            a[4] += v.x; a[5] += v.y; a[6] += v.z; a[7] += v.w;
        }
    } else {
        for (int r = r0; r < r1; ++r)
            for (int e = 0; e < 8 && c0 + e < N; ++e) a[e] += to_f32(Y[(int64_t)r * ld + c0 + e]);
    }
    for (int e = 0; e < 8 && c0 + e < N; ++e) part[(int64_t)blockIdx.y * N + c0 + e] = a[e];
}

int colsum_num_partials(int M) { return ceil_div(M, CS_ROWS); }

void colsum_rows(bool y_bf, const void* Y, int64_t ld, int M, int N, float* partial, hipStream_t s) {
    const int np = ceil_div(M, CS_ROWS);
    dim3 grid(ceil_div(N, 64 * 8), np);
    const bool vec = (ld % 8) == 0 && ((uintptr_t)Y % 16) == 0;
    if (y_bf && vec) colsum_kernel<bf16><<<grid, 64, 0, s>>>((const bf16*)Y, ld, M, N, partial);
    else if (!y_bf && vec) colsum_kernel<float><<<grid, 64, 0, s>>>((const float*)Y, ld, M, N, partial);
    else {
        // unaligned fallback: one column per thread
        if (y_bf) colsum_scalar_kernel<bf16><<<dim3(ceil_div(N, 256), np), 256, 0, s>>>((const bf16*)Y, ld, M, N, partial);
        else colsum_scalar_kernel<float><<<dim3(ceil_div(N, 256), np), 256, 0, s>>>((const float*)Y, ld, M, N, partial);
    }
}

void colsum(bool y_bf, const void* Y, int64_t ld, int M, int N, float* out, float* partial, hipStream_t s) {
    const int np = ceil_div(M, CS_ROWS);
    colsum_rows(y_bf, Y, ld, M, N, partial, s);
    reduce_partials(partial, np, N, 1, partial + (size_t)np * N, out, nullptr, nullptr, s);
}

// =====================================================================
// fused softmax cross-entropy, forward + backward, in place
// =====================================================================

template <typename T>
__global__ __launch_bounds__(256) void cross_entropy_kernel(T* z, const int32_t* y, float* row_loss, int Vp,
                                                            float gscale, float cap, int32_t* err) {
    __shared__ float smx[4], ssm[4];
    const int row = blockIdx.x;
    T* zr = z + (int64_t)row * Vp;
    const int tgt = y[row];
    const bool valid = tgt >= 0 && tgt < Vp;
    const float icap = cap > 0.f ? 1.0f / cap : 0.f;
    const float L2E = 1.4426950408889634f;
    float mx = -INFINITY, sm = 0.f;   // running max and sum of exp2((z - mx) log2e)
    for (int v = threadIdx.x; v < Vp; v += 256) {
        float zz = to_f32(zr[v]);
        if (cap > 0.f) zz = cap * tanhf(zz * icap);
        zz *= L2E;
        if (zz > mx) { sm = sm * exp2f(mx - zz) + 1.0f; mx = zz; }
        else sm += exp2f(zz - mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(mx, o, 64), s2 = __shfl_xor(sm, o, 64);
        float mn = fmaxf(mx, m2);
        sm = (mx == -INFINITY ? 0.f : sm * exp2f(mx - mn)) + (m2 == -INFINITY ? 0.f : s2 * exp2f(m2 - mn));
        mx = mn;
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { smx[w] = mx; ssm[w] = sm; }
    __syncthreads();
    float gm = fmaxf(fmaxf(smx[0], smx[1]), fmaxf(smx[2], smx[3]));
    float gs = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) gs += smx[i] == -INFINITY ? 0.f : ssm[i] * exp2f(smx[i] - gm);
    const float lse2 = gm + log2f(gs);   // log2-domain logsumexp
    if (threadIdx.x == 0) {
        float loss = 0.f;
        if (valid) {
            float zy = to_f32(zr[tgt]);
            if (cap > 0.f) zy = cap * tanhf(zy * icap);
            loss = lse2 * 0.6931471805599453f - zy;
        } else {
            *err = 1;
        }
        row_loss[row] = loss;
    }
    __syncthreads();   // the target logit is read before any thread overwrites it
    for (int v = threadIdx.x; v < Vp; v += 256) {
        float g = 0.f;
        if (valid) {
            float zz = to_f32(zr[v]);
            float th = 0.f;
            if (cap > 0.f) { th = tanhf(zz * icap); zz = cap * th; }
            float p = exp2f(zz * L2E - lse2);
            g = (p - (v == tgt ? 1.0f : 0.0f)) * gscale;
            if (cap > 0.f) g *= (1.0f - th * th);
        }
        zr[v] = from_f32<T>(g);
    }
}

// bf16 logits with Vp % 8 == 0: the row is read once into registers (CPT
// 16-byte chunks per thread), reduced (max, then sum of exp), and the gradient
// is written back from registers: one read and one write of the row.
typedef uint32_t ce_u32x4 __attribute__((ext_vector_type(4)));

GPT_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
GPT_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// CAP: logit softcap on (a template parameter, so the plain path does not
// carry the capped path's registers)
template <int CPT, bool CAP>
__global__ __launch_bounds__(256) void cross_entropy_reg_kernel(bf16* z, const int32_t* y, float* row_loss, int Vp,
                                                                float gscale, float cap, int32_t* err) {
    __shared__ float sred[8];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    bf16* zr = z + (int64_t)row * Vp;
    const int nch = Vp >> 3;
    const int tgt = y[row];
    const bool valid = tgt >= 0 && tgt < Vp;
    const float icap = CAP ? 1.0f / cap : 0.f;
    const float L2E = 1.4426950408889634f;
    ce_u32x4 v[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int idx = tid + 256 * c;
        ce_u32x4 zero = {0u, 0u, 0u, 0u};
        v[c] = idx < nch ? *reinterpret_cast<const ce_u32x4*>(zr + 8 * idx) : zero;
    }
    auto raw = [&](int c, int e) {   // logit as stored
        const uint32_t wd = v[c][e >> 1];
        return (e & 1) ? bf_hi(wd) : bf_lo(wd);
    };
    auto capped = [&](float x) { return CAP ? cap * tanh_exp2(x * icap) : x; };
    // the target logit, read before any thread overwrites the row (the barriers
    // below wait for it)
    const float zt_raw = (tid == 0 && valid) ? (float)zr[tgt] : 0.f;
    // pass 1: maximum (of the capped logits: the cap is monotone, so cap(max))
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < CPT; ++c)
        if (tid + 256 * c < nch)
#pragma unroll
            for (int e = 0; e < 8; e += 2) mx = fmaxf(mx, fmaxf(raw(c, e), raw(c, e + 1)));
    // the unpacked logits of this pass are recomputed in the next one rather
    // than kept live across it (200 floats per thread would halve occupancy)
#pragma unroll
    for (int c = 0; c < CPT; ++c) asm volatile("" : "+v"(v[c]));
    mx = wave_max(mx);
    if (lane == 0) sred[w] = mx;
    __syncthreads();
    const float gm = capped(fmaxf(fmaxf(sred[0], sred[1]), fmaxf(sred[2], sred[3]))) * L2E;   // log2 units
    // pass 2: sum of exp (log2 units: 2^(x log2 e - gm))
    float sm = 0.f;
    if constexpr (CAP) {
#pragma unroll
        for (int c = 0; c < CPT; ++c)
            if (tid + 256 * c < nch)
#pragma unroll
                for (int e = 0; e < 8; ++e) sm += __builtin_amdgcn_exp2f(fmaf(capped(raw(c, e)), L2E, -gm));
    } else {
        // without the cap each chunk's exponentials replace its logits (bf16,
        // in the same registers), so the gradient pass needs one multiply per
        // element instead of a second exponential
#pragma unroll
        for (int c = 0; c < CPT; ++c)
            if (tid + 256 * c < nch) {
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(raw(c, 2 * e2), L2E, -gm));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(raw(c, 2 * e2 + 1), L2E, -gm));
                    sm += p0 + p1;
                    const bf16 lo = (bf16)p0, hi = (bf16)p1;
                    v[c][e2] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                               ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
            }
    }
    sm = wave_sum(sm);
    if (lane == 0) sred[4 + w] = sm;
    __syncthreads();
    const float lse2 = gm + log2f((sred[4] + sred[5]) + (sred[6] + sred[7]));
    // pass 3: gradient softmax * gscale (times 1 - tanh^2 under the cap), written
    // over the row with non-temporal stores (the row is not read again by this
    // kernel; the products that read it stream 1.6 GB); the target's -gscale is
    // applied by thread 0 afterwards
    const float gs = valid ? gscale : 0.f;
    // exp2(x log2e - gm) -> softmax * gscale
    const float rescale = __builtin_amdgcn_exp2f(gm - lse2) * gs;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const int idx = tid + 256 * c;
        if (idx >= nch) continue;
        ce_u32x4 o;
        if constexpr (!CAP) {
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const bf16 lo = (bf16)(bf_lo(v[c][e2]) * rescale), hi = (bf16)(bf_hi(v[c][e2]) * rescale);
                o[e2] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            __builtin_nontemporal_store(o, reinterpret_cast<ce_u32x4*>(zr + 8 * idx));
            continue;
        }
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            float gpair[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float x = raw(c, 2 * e2 + h);
                if constexpr (CAP) {
                    const float th = tanh_exp2(x * icap);
                    gpair[h] = __builtin_amdgcn_exp2f(fmaf(cap * th, L2E, -lse2)) * gs * (1.0f - th * th);
                } else {
                    gpair[h] = __builtin_amdgcn_exp2f(fmaf(x, L2E, -lse2)) * gs;
                }
            }
            const bf16 lo = (bf16)gpair[0], hi = (bf16)gpair[1];
            o[e2] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        __builtin_nontemporal_store(o, reinterpret_cast<ce_u32x4*>(zr + 8 * idx));
    }
    // the target: loss lse - z_t, and its gradient element (p_t - 1) * gscale (times
    // 1 - tanh^2 under the cap), written after every thread's chunk stores
    __syncthreads();
    if (tid == 0) {
        float loss = 0.f;
        if (valid) {
            float th = 0.f, zt = zt_raw;
            if constexpr (CAP) { th = tanh_exp2(zt * icap); zt = cap * th; }
            loss = lse2 * 0.6931471805599453f - zt;
            float g = (__builtin_amdgcn_exp2f(fmaf(zt, L2E, -lse2)) - 1.0f) * gscale;
            if constexpr (CAP) g *= 1.0f - th * th;
            zr[tgt] = (bf16)g;
        } else {
            *err = 1;
        }
        row_loss[row] = loss;
    }
}

void cross_entropy(bool bf, void* z, const int32_t* y, float* row_loss, int M, int Vp, float gscale, float cap,
                   int32_t* err, hipStream_t s) {
    const int nch = Vp / 8;
    if (bf && Vp % 8 == 0 && ((uintptr_t)z % 16) == 0 && nch <= 32 * 256) {
        const int cpt = ceil_div(nch, 256);
        bf16* zb = (bf16*)z;
        auto run = [&](auto cpt_c) {
            constexpr int C = decltype(cpt_c)::value;
            if (cap > 0.f) cross_entropy_reg_kernel<C, true><<<M, 256, 0, s>>>(zb, y, row_loss, Vp, gscale, cap, err);
            else cross_entropy_reg_kernel<C, false><<<M, 256, 0, s>>>(zb, y, row_loss, Vp, gscale, cap, err);
        };
        if (cpt <= 4) run(std::integral_constant<int, 4>{});
        else if (cpt <= 8) run(std::integral_constant<int, 8>{});
        else if (cpt <= 16) run(std::integral_constant<int, 16>{});
        else if (cpt <= 25) run(std::integral_constant<int, 25>{});
        else run(std::integral_constant<int, 32>{});
        return;
    }
    if (bf) cross_entropy_kernel<bf16><<<M, 256, 0, s>>>((bf16*)z, y, row_loss, Vp, gscale, cap, err);
    else cross_entropy_kernel<float><<<M, 256, 0, s>>>((float*)z, y, row_loss, Vp, gscale, cap, err);
}

__global__ __launch_bounds__(256) void mean_loss_kernel(const float* rl, int M, float* out, float* sum, int first) {
    __shared__ double sh[4];
    double a = 0.0;
    int i = threadIdx.x;
    // eight rows loaded together, added in row order
    for (; i + 7 * 256 < M; i += 8 * 256) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = rl[i + u * 256];
#pragma unroll
        for (int u = 0; u < 8; ++u) a += v[u];
    }
    for (; i < M; i += 256) a += rl[i];
    a = wave_sum_d(a);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = ((sh[0] + sh[1]) + sh[2]) + sh[3];
        float mval = (float)(t / M);
        *out = mval;
        *sum = first ? mval : *sum + mval;
    }
}
void mean_loss(const float* row_loss, int M, float* loss_out, float* loss_sum, hipStream_t s, bool first) {
    mean_loss_kernel<<<1, 256, 0, s>>>(row_loss, M, loss_out, loss_sum, first ? 1 : 0);
}

// =====================================================================
// attention row dots D = rowsum(dO * O), per head
// =====================================================================

template <typename T>
__global__ __launch_bounds__(256) void attn_rowdot_kernel(const T* dO, const T* O, float* D, int B, int T_, int H,
                                                          int hd) {
    int idx = blockIdx.x * 256 + threadIdx.x;   // (m, h)
    if (idx >= B * T_ * H) return;
    int m = idx / H, h = idx % H;
    int b = m / T_, t = m % T_;
    const int64_t off = (int64_t)m * H * hd + (int64_t)h * hd;
    float a = 0.f;
    for (int c = 0; c < hd; c += 4) {
        float4 x = load4(dO + off + c), y = load4(O + off + c);
        a += (x.x * y.x + x.y * y.y) + (x.z * y.z + x.w * y.w);
    }
    D[((int64_t)b * H + h) * T_ + t] = a;
}

void attn_rowdot(bool bf, const void* dO, const void* O, float* D, int B, int T, int H, int hd, hipStream_t s) {
    int n = B * T * H;
    if (bf) attn_rowdot_kernel<bf16><<<ceil_div(n, 256), 256, 0, s>>>((const bf16*)dO, (const bf16*)O, D, B, T, H, hd);
    else attn_rowdot_kernel<float><<<ceil_div(n, 256), 256, 0, s>>>((const float*)dO, (const float*)O, D, B, T, H, hd);
}

// =====================================================================
// q/k RMS normalisation + rotary positions. Portable form: one wavefront per
// (row, head, q|k), lane i < hd/2 holding the rotate-half pair (i, i + hd/2);
// bf16 with hd in {16, 32, 64, 128} takes the vectorised form below.
// =====================================================================

template <typename T>
__global__ __launch_bounds__(256) void qk_prep_fwd_kernel(const T* qkv, T* out, const float* cos_t,
                                                          const float* sin_t, int M, int T_, int H, int hd,
                                                          int norm, int rope, float eps, int pos0) {
    int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wid >= M * H * 2) return;
    int which = wid & 1, mh = wid >> 1, m = mh / H, h = mh % H;
    int half = hd >> 1, d = H * hd;
    const T* src = qkv + (int64_t)m * 3 * d + which * d + h * hd;
    T* dst = out + (int64_t)m * 2 * d + which * d + h * hd;
    bool act = lane < half;
    float a = act ? to_f32(src[lane]) : 0.f, b = act ? to_f32(src[lane + half]) : 0.f;
    if (norm) {
        float ss = wave_sum(a * a + b * b);
        float r = 1.0f / sqrtf(ss / hd + eps);
        a *= r; b *= r;
    }
    if (rope && act) {
        int t = pos0 + m % T_;
        float c = cos_t[t * half + lane], sn = sin_t[t * half + lane];
        float na = a * c - b * sn, nb = a * sn + b * c;
        a = na; b = nb;
    }
    if (act) { dst[lane] = from_f32<T>(a); dst[lane + half] = from_f32<T>(b); }
}

template <typename T>
__global__ __launch_bounds__(256) void qk_prep_bwd_kernel(const T* qkv, T* dqkv, const float* cos_t,
                                                          const float* sin_t, int M, int T_, int H, int hd,
                                                          int norm, int rope, float eps) {
    int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (wid >= M * H * 2) return;
    int which = wid & 1, mh = wid >> 1, m = mh / H, h = mh % H;
    int half = hd >> 1, d = H * hd;
    const T* src = qkv + (int64_t)m * 3 * d + which * d + h * hd;
    T* g = dqkv + (int64_t)m * 3 * d + which * d + h * hd;
    bool act = lane < half;
    float ga = act ? to_f32(g[lane]) : 0.f, gb = act ? to_f32(g[lane + half]) : 0.f;
    if (rope && act) {
        int t = m % T_;
        float c = cos_t[t * half + lane], sn = sin_t[t * half + lane];
        float na = ga * c + gb * sn, nb = -ga * sn + gb * c;
        ga = na; gb = nb;
    }
    if (norm) {
        float a = act ? to_f32(src[lane]) : 0.f, b = act ? to_f32(src[lane + half]) : 0.f;
        float ss = wave_sum(a * a + b * b);
        float r = 1.0f / sqrtf(ss / hd + eps);
        float ya = a * r, yb = b * r;
        float dot = wave_sum(ga * ya + gb * yb) / hd;
        ga = r * (ga - ya * dot);
        gb = r * (gb - yb * dot);
    }
    if (act) { g[lane] = from_f32<T>(ga); g[lane + half] = from_f32<T>(gb); }
}

// bf16 with hd a multiple of 16: LPU = hd / 16 lanes per (row, head, q|k),
// lane j holding elements 8j .. 8j+7 of the first half and their rotate-half
// partners 8j + hd/2 .. in 16-byte pieces (the rotation needs no exchange
// between lanes; the RMS sum is a butterfly over the unit's lanes)
template <int LPU>
GPT_DEV float unit_sum(float v) {
#pragma unroll
    for (int o = 1; o < LPU; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}
GPT_DEV void unpack8(const bf16x8& v, float (&f)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
}
GPT_DEV bf16x8 pack8(const float (&f)[8]) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)f[e];
    return v;
}
GPT_DEV void load8f(const float* p, float (&f)[8]) {
    const float4 u = reinterpret_cast<const float4*>(p)[0], w = reinterpret_cast<const float4*>(p)[1];
    f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w; f[4] = w.x; f[5] = w.y; f[6] = w.z; f[7] = w.w;
}

template <int LPU>
__global__ __launch_bounds__(256) void qk_prep_fwd_vec_kernel(const bf16* qkv, bf16* out, const float* cos_t,
                                                              const float* sin_t, int M, int T_, int H, int norm,
                                                              int rope, float eps, int pos0) {
    constexpr int HD = 16 * LPU, HALF = HD / 2;
    const int64_t u = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPU;   // (row, head, q|k)
    const int j = threadIdx.x % LPU;
    if (u >= (int64_t)M * H * 2) return;   // whole units: every lane of a unit returns together
    const int which = (int)(u & 1), mh = (int)(u >> 1), m = mh / H, h = mh % H, d = H * HD;
    const bf16* src = qkv + (int64_t)m * 3 * d + which * d + h * HD + 8 * j;
    bf16* dst = out + (int64_t)m * 2 * d + which * d + h * HD + 8 * j;
    float a[8], b[8];
    unpack8(*reinterpret_cast<const bf16x8*>(src), a);
    unpack8(*reinterpret_cast<const bf16x8*>(src + HALF), b);
    if (norm) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += a[e] * a[e] + b[e] * b[e];
        const float r = 1.0f / sqrtf(unit_sum<LPU>(ss) / HD + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) { a[e] *= r; b[e] *= r; }
    }
    if (rope) {
        const int t = pos0 + m % T_;
        float c[8], sn[8];
        load8f(cos_t + (int64_t)t * HALF + 8 * j, c);
        load8f(sin_t + (int64_t)t * HALF + 8 * j, sn);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float na = a[e] * c[e] - b[e] * sn[e], nb = a[e] * sn[e] + b[e] * c[e];
            a[e] = na; b[e] = nb;
        }
    }
    *reinterpret_cast<bf16x8*>(dst) = pack8(a);
    *reinterpret_cast<bf16x8*>(dst + HALF) = pack8(b);
}

template <int LPU>
__global__ __launch_bounds__(256) void qk_prep_bwd_vec_kernel(const bf16* qkv, bf16* dqkv, const float* cos_t,
                                                              const float* sin_t, int M, int T_, int H, int norm,
                                                              int rope, float eps) {
    constexpr int HD = 16 * LPU, HALF = HD / 2;
    const int64_t u = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPU;
    const int j = threadIdx.x % LPU;
    if (u >= (int64_t)M * H * 2) return;
    const int which = (int)(u & 1), mh = (int)(u >> 1), m = mh / H, h = mh % H, d = H * HD;
    const bf16* src = qkv + (int64_t)m * 3 * d + which * d + h * HD + 8 * j;
    bf16* g = dqkv + (int64_t)m * 3 * d + which * d + h * HD + 8 * j;
    float ga[8], gb[8];
    unpack8(*reinterpret_cast<const bf16x8*>(g), ga);
    unpack8(*reinterpret_cast<const bf16x8*>(g + HALF), gb);
    float a[8], b[8];
    if (norm) {
        unpack8(*reinterpret_cast<const bf16x8*>(src), a);
        unpack8(*reinterpret_cast<const bf16x8*>(src + HALF), b);
    }
    if (rope) {
        const int t = m % T_;
        float c[8], sn[8];
        load8f(cos_t + (int64_t)t * HALF + 8 * j, c);
        load8f(sin_t + (int64_t)t * HALF + 8 * j, sn);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float na = ga[e] * c[e] + gb[e] * sn[e], nb = -ga[e] * sn[e] + gb[e] * c[e];
            ga[e] = na; gb[e] = nb;
        }
    }
    if (norm) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += a[e] * a[e] + b[e] * b[e];
        const float r = 1.0f / sqrtf(unit_sum<LPU>(ss) / HD + eps);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += ga[e] * (a[e] * r) + gb[e] * (b[e] * r);
        dot = unit_sum<LPU>(dot) / HD;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ga[e] = r * (ga[e] - a[e] * r * dot);
            gb[e] = r * (gb[e] - b[e] * r * dot);
        }
    }
    *reinterpret_cast<bf16x8*>(g) = pack8(ga);
    *reinterpret_cast<bf16x8*>(g + HALF) = pack8(gb);
}

template <template <int> class K, typename... A>
static bool qk_vec_launch(int hd, int64_t units, hipStream_t s, A... args) {
    const unsigned grid = (unsigned)ceil_div(units * (hd / 16), 256);
    switch (hd) {
        case 16: K<1>::launch(grid, s, args...); return true;
        case 32: K<2>::launch(grid, s, args...); return true;
        case 64: K<4>::launch(grid, s, args...); return true;
        case 128: K<8>::launch(grid, s, args...); return true;
        default: return false;
    }
}
template <int LPU>
struct QkFwdVec {
    template <typename... A>
    static void launch(unsigned grid, hipStream_t s, A... args) { qk_prep_fwd_vec_kernel<LPU><<<grid, 256, 0, s>>>(args...); }
};
template <int LPU>
struct QkBwdVec {
    template <typename... A>
    static void launch(unsigned grid, hipStream_t s, A... args) { qk_prep_bwd_vec_kernel<LPU><<<grid, 256, 0, s>>>(args...); }
};

void qk_prep_fwd(bool bf, const void* qkv, void* out, const float* cos_t, const float* sin_t, int M, int T, int H,
                 int hd, int norm, int rope, float eps, hipStream_t s, int pos0) {
    int grid = ceil_div((int64_t)M * H * 2, 4);
    if (bf && qk_vec_launch<QkFwdVec>(hd, (int64_t)M * H * 2, s, (const bf16*)qkv, (bf16*)out, cos_t, sin_t, M, T, H,
                                      norm, rope, eps, pos0))
        return;
    if (bf)
        qk_prep_fwd_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)qkv, (bf16*)out, cos_t, sin_t, M, T, H, hd, norm,
                                                      rope, eps, pos0);
    else
        qk_prep_fwd_kernel<float><<<grid, 256, 0, s>>>((const float*)qkv, (float*)out, cos_t, sin_t, M, T, H, hd,
                                                       norm, rope, eps, pos0);
}
void qk_prep_bwd(bool bf, const void* qkv, void* dqkv, const float* cos_t, const float* sin_t, int M, int T, int H,
                 int hd, int norm, int rope, float eps, hipStream_t s) {
    int grid = ceil_div((int64_t)M * H * 2, 4);
    if (bf && qk_vec_launch<QkBwdVec>(hd, (int64_t)M * H * 2, s, (const bf16*)qkv, (bf16*)dqkv, cos_t, sin_t, M, T, H,
                                      norm, rope, eps))
        return;
    if (bf)
        qk_prep_bwd_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)qkv, (bf16*)dqkv, cos_t, sin_t, M, T, H, hd, norm,
                                                      rope, eps);
    else
        qk_prep_bwd_kernel<float><<<grid, 256, 0, s>>>((const float*)qkv, (float*)dqkv, cos_t, sin_t, M, T, H, hd,
                                                       norm, rope, eps);
}

// =====================================================================
// global gradient norm (two deterministic passes in double) and AdamW
// =====================================================================

constexpr int GN_BLOCKS = 1024;

// Four independent loads and sums per iteration keep enough bytes in flight
// for HBM (one float4 per thread left it latency-bound at about 58% of peak);
// the order of the additions is fixed, so the result is deterministic.
__global__ __launch_bounds__(256) void grad_norm_partial_kernel(const float* g, int64_t n, double* part) {
    __shared__ double sh[4];
    auto sq = [](const float4 v) {
        return (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
    };
    const int64_t n4 = n >> 2, stride = (int64_t)GN_BLOCKS * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    for (; i + 3 * stride < n4; i += 4 * stride) {
        const float4 v0 = load4(g + 4 * i), v1 = load4(g + 4 * (i + stride)), v2 = load4(g + 4 * (i + 2 * stride)),
                     v3 = load4(g + 4 * (i + 3 * stride));
        a0 += sq(v0);
        a1 += sq(v1);
        a2 += sq(v2);
        a3 += sq(v3);
    }
    for (; i < n4; i += stride) a0 += sq(load4(g + 4 * i));
    double a = (a0 + a1) + (a2 + a3);
    if (blockIdx.x == 0)
        for (int64_t i = 4 * n4 + threadIdx.x; i < n; i += 256) a += (double)g[i] * g[i];
    a = wave_sum_d(a);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = ((sh[0] + sh[1]) + sh[2]) + sh[3];
}

__global__ __launch_bounds__(256) void grad_norm_final_kernel(const double* part, float* norm_out, float* coef_out,
                                                              int32_t* skip, const int32_t* id_err, float max_norm) {
    __shared__ double sh[4];
    double a = 0.0;
    for (int i = threadIdx.x; i < GN_BLOCKS; i += 256) a += part[i];
    a = wave_sum_d(a);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = a;
    __syncthreads();
    if (threadIdx.x == 0) {
        double nrm = sqrt(((sh[0] + sh[1]) + sh[2]) + sh[3]);
        // skip the update for a non-finite norm, or while an out-of-range
        // token or target id is pending (its rows contributed no gradient)
        bool bad = !isfinite(nrm) || (id_err && *id_err);
        double c = (double)max_norm / (nrm + 1e-6);
        *norm_out = (float)nrm;
        *coef_out = bad ? 0.f : (float)(c < 1.0 ? c : 1.0);
        *skip = bad ? 1 : 0;
    }
}

void grad_norm(const float* g, int64_t n, double* partial, float* norm_out, float* coef_out, int32_t* skip,
               const int32_t* id_err, float max_norm, hipStream_t s) {
    grad_norm_partial_kernel<<<GN_BLOCKS, 256, 0, s>>>(g, n, partial);
    grad_norm_final_kernel<<<1, 256, 0, s>>>(partial, norm_out, coef_out, skip, id_err, max_norm);
}

GPT_DEV void adamw4(float4& pp, const float4& gg, float4& mm, float4& vv, bool decayed, float c, float dec, float lr,
                    float b1, float b2, float eps, float rbc1, float rbc2) {
    float* pe = &pp.x; const float* ge = &gg.x; float* me = &mm.x; float* ve = &vv.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float gc = ge[e] * c;
        me[e] = b1 * me[e] + (1.0f - b1) * gc;
        ve[e] = b2 * ve[e] + (1.0f - b2) * gc * gc;
        const float pv = decayed ? pe[e] * dec : pe[e];
        pe[e] = pv - lr * (me[e] * rbc1) / (sqrtf(ve[e] * rbc2) + eps);
    }
}

// One group of four parameters per thread, one pass over the grid (every load
// of the group issued before its stores; the parameters, moments and bf16
// copy are written with non-temporal stores: nothing reads them again before
// the next step).
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ p, const float* __restrict__ g,
                                                    float* __restrict__ m, float* __restrict__ v, bf16* __restrict__ wbf,
                                                    int64_t n4, int64_t nd4, const float* coef_p,
                                                    const int32_t* nonfinite, float lr, float b1, float b2,
                                                    float eps, float wd, float rbc1, float rbc2) {
    if (*nonfinite) return;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const float c = *coef_p;
    const float dec = 1.0f - lr * wd;
    float4 p0 = load4(p + 4 * i), g0 = load4(g + 4 * i), m0 = load4(m + 4 * i), v0 = load4(v + 4 * i);
    adamw4(p0, g0, m0, v0, i < nd4, c, dec, lr, b1, b2, eps, rbc1, rbc2);
    auto nt4 = [](float* dst, const float4& x) {
        const f32x4 t = {x.x, x.y, x.z, x.w};
        __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(dst));
    };
    nt4(p + 4 * i, p0);
    nt4(m + 4 * i, m0);
    nt4(v + 4 * i, v0);
    if (i < nd4 && wbf) {
        bf16x4 o;
        o[0] = (bf16)p0.x; o[1] = (bf16)p0.y; o[2] = (bf16)p0.z; o[3] = (bf16)p0.w;
        __builtin_nontemporal_store(o, reinterpret_cast<bf16x4*>(wbf + 4 * i));
    }
}

void adamw(float* p, const float* g, float* m, float* v, void* wbf, int64_t n, int64_t n_decay, const float* coef,
           const int32_t* nonfinite, float lr, float b1, float b2, float eps, float wd, float rbc1, float rbc2,
           hipStream_t s) {
    int64_t n4 = n / 4;
    unsigned grid = (unsigned)((n4 + 255) / 256);
    adamw_kernel<<<grid, 256, 0, s>>>(p, g, m, v, (bf16*)wbf, n4, n_decay / 4, coef, nonfinite, lr, b1, b2, eps, wd,
                                      rbc1, rbc2);
}

// =====================================================================
// FP8 head: per-tensor e4m3 quantisation (OCP E4M3, largest finite 448)
// =====================================================================

constexpr int AMAX_BLOCKS = 1024;

__global__ __launch_bounds__(256) void amax_bf16_kernel(const bf16* __restrict__ x, int64_t n8, float* part) {
    __shared__ float sh[4];
    float m = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)AMAX_BLOCKS * 256) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + 8 * i);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)v[e]));
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

__global__ __launch_bounds__(256) void amax_final_kernel(const float* part, float* scale, float* inv) {
    __shared__ float sh[4];
    float m = 0.f;
    for (int i = threadIdx.x; i < AMAX_BLOCKS; i += 256) m = fmaxf(m, part[i]);
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float a = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
        const float sc = a > 0.f ? 448.0f / a : 1.0f;
        *scale = sc;
        *inv = 1.0f / sc;
    }
}

// eight values per thread: fp32 product with the scale, clamped to [-448, 448],
// converted in pairs to e4m3 (round to nearest even) by v_cvt_pk_fp8_f32
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const bf16* __restrict__ x, int64_t n8,
                                                            const float* __restrict__ scale, uint8_t* __restrict__ q) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n8) return;
    const float sc = *scale;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + 8 * i);
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = fminf(fmaxf((float)v[e] * sc, -448.0f), 448.0f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
    *reinterpret_cast<int2*>(q + 8 * i) = make_int2(lo, hi);
}

void quantize_e4m3(const void* x, int64_t n, uint8_t* q, float* scale, float* inv, float* part, hipStream_t s) {
    const int64_t n8 = n / 8;
    amax_bf16_kernel<<<AMAX_BLOCKS, 256, 0, s>>>((const bf16*)x, n8, part);
    amax_final_kernel<<<1, 256, 0, s>>>(part, scale, inv);
    quantize_e4m3_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>((const bf16*)x, n8, scale, q);
}

}  // namespace gk
