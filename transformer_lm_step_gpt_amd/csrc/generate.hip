// Decode-shaped kernels of autoregressive sampling with a key/value cache:
// one new token per sequence and step ("Un GPT desde cero + nanoGPT" 2.1,
// generate; the lecture notes' "Генерация и устройство", top-k sampling).
//
//   gen_embed      x[b] = wte[token at pos] + wpe[pos] for each sequence b
//   cache_put      rows of k or v (from the qkv / q,k buffers) into the cache
//                  [B, Tmax, d] of one layer at positions t0 .. (prefill)
//   gen_attention  writes the step's key and value rows into the caches, then
//                  one query per (sequence, head) against the cached keys and
//                  values 0 .. pos (or the last `window` of them)
//   gen_sample     one draw per sequence from the last position's logits:
//                  softcap, temperature, top-k, inverse CDF in token order
//                  (a gathered top-k path and a general token-order path)
//   skinny_gemm    the products of a decode step (M = B <= 16 rows): each
//                  wave streams 16 weight rows and multiplies them with the
//                  activations held in LDS (v_mfma_f32_16x16x32_bf16)
#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

#include <cfloat>
#include <climits>

namespace gk {

// ---------------------------------------------------------------- helpers

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds on a 4-word
// counter with a 2-word key advanced by the Weyl constants between rounds.
GPT_DEV void gen_philox(uint64_t c[4], uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r) { k0 += W0; k1 += W1; }
        const uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
        const uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
        const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
    }
}

constexpr uint64_t SAMPLE_STREAM = 0x73616D706C65ull;   // key word 1 of the sampling draws

// Monotone map of a float onto uint32 (larger float -> larger key).
GPT_DEV uint32_t order_key(float z) {
    const uint32_t u = __float_as_uint(z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide reductions and scans over NT threads (NT a multiple of 64, at
// most 1024), in a fixed order. `sh` holds at least NT / 64 + 1 slots.
template <int NT>
GPT_DEV float block_max_f(float v, float* sh) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float r = sh[0];
    for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, sh[i]);
    return r;
}
template <int NT>
GPT_DEV float block_sum_f(float v, float* sh) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float r = sh[0];
    for (int i = 1; i < NT / 64; ++i) r += sh[i];
    return r;
}
template <int NT>
GPT_DEV int block_sum_i(int v, int* sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    int r = 0;
    for (int i = 0; i < NT / 64; ++i) r += sh[i];
    return r;
}
template <int NT>
GPT_DEV int block_max_i(int v, int* sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    int r = sh[0];
    for (int i = 1; i < NT / 64; ++i) r = max(r, sh[i]);
    return r;
}
// exclusive prefix sum over the threads in thread order; *total receives the sum
template <int NT, typename V>
GPT_DEV V block_excl_scan(V v, V* sh, V* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    V incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const V u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
    __syncthreads();
    if (lane == 63) sh[w] = incl;
    __syncthreads();
    V off = 0, tot = 0;
    for (int i = 0; i < NT / 64; ++i) {
        if (i < w) off += sh[i];
        tot += sh[i];
    }
    *total = tot;
    return off + incl - v;
}

// ---------------------------------------------------------------- embedding of one token per sequence

__global__ __launch_bounds__(256) void gen_embed_kernel(const int32_t* seq, int64_t ld, int pos, const float* wte,
                                                        const float* wpe, float* x, int B, int d, int Vp,
                                                        int32_t* err) {
    const int dq = d >> 2;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= B * dq) return;
    const int b = idx / dq, c = (idx % dq) * 4;
    const int id = seq[(int64_t)b * ld + pos];
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (id >= 0 && id < Vp) v = load4(wte + (int64_t)id * d + c);
    else if (c == 0) *err = 1;
    if (wpe) {
        const float4 p = load4(wpe + (int64_t)pos * d + c);
        v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
    }
    store4(x + (int64_t)b * d + c, v);
}

void gen_embed(const int32_t* seq, int64_t ld, int pos, const float* wte, const float* wpe, float* x, int B, int d,
               int Vp, int32_t* err, hipStream_t s) {
    const int n = B * (d / 4);
    gen_embed_kernel<<<ceil_div(n, 256), 256, 0, s>>>(seq, ld, pos, wte, wpe, x, B, d, Vp, err);
}

// ---------------------------------------------------------------- cache rows

// dst[(b Tmax + t0 + t) d + c] = src[(b nt + t) src_ld + c]; 16 bytes per thread
template <typename T>
__global__ __launch_bounds__(256) void cache_put_kernel(const T* src, int64_t src_ld, T* dst, int B, int nt, int Tmax,
                                                        int t0, int d) {
    constexpr int E = 16 / sizeof(T);
    const int cpr = d / E;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)B * nt * cpr) return;
    const int c = (int)(idx % cpr) * E;
    const int64_t r = idx / cpr;
    const int t = (int)(r % nt), b = (int)(r / nt);
    const uint4 v = *reinterpret_cast<const uint4*>(src + ((int64_t)b * nt + t) * src_ld + c);
    *reinterpret_cast<uint4*>(dst + ((int64_t)b * Tmax + t0 + t) * d + c) = v;
}

void cache_put(bool bf, const void* src, int64_t src_ld, void* dst, int B, int nt, int Tmax, int t0, int d,
               hipStream_t s) {
    const int64_t n = (int64_t)B * nt * (d / (bf ? 8 : 4));
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (!grid) return;
    if (bf) cache_put_kernel<bf16><<<grid, 256, 0, s>>>((const bf16*)src, src_ld, (bf16*)dst, B, nt, Tmax, t0, d);
    else cache_put_kernel<float><<<grid, 256, 0, s>>>((const float*)src, src_ld, (float*)dst, B, nt, Tmax, t0, d);
}

// ---------------------------------------------------------------- attention of one query against the cache

// One workgroup per (sequence, head): the new key and value rows of the
// head are copied into the caches at position pos (the barrier below makes
// them visible to the whole workgroup); the scores of the query against keys
// j0 .. pos in LDS (one key per thread and pass), softmax in fp32; then
// out[c] = sum_j p_j v_j[c] with thread (g, ch) accumulating the 16-byte
// chunk ch of the value rows j = g, g + KG, ... (the first GA_VPRE of them
// loaded before the softmax, beside the keys), and the KG partial rows
// summed in a fixed order.
constexpr int GA_VPRE = 8;

template <typename T>
__global__ __launch_bounds__(256) void gen_attention_kernel(const T* q, int64_t ldq, const T* knew, int64_t ldk,
                                                            const T* vnew, int64_t ldv, T* kc, T* vc, T* out, int H,
                                                            int hd, int pos, int Tmax, int window, float scale) {
    extern __shared__ float sc[];   // [pos + 1] scores, then weights; then the partial output rows
    __shared__ float qs[128];
    __shared__ float rsh[16];
    constexpr int E = 16 / sizeof(T);   // elements per 16-byte chunk
    const int b = blockIdx.x / H, h = blockIdx.x % H, tid = threadIdx.x;
    const int d = H * hd;
    const int j0 = (window > 0 && pos - window + 1 > 0) ? pos - window + 1 : 0;
    const int n = pos + 1 - j0;
    if (tid < hd) {
        qs[tid] = to_f32(q[(int64_t)b * ldq + h * hd + tid]);
        const int64_t o = ((int64_t)b * Tmax + pos) * d + h * hd + tid;
        kc[o] = knew[(int64_t)b * ldk + h * hd + tid];
        vc[o] = vnew[(int64_t)b * ldv + h * hd + tid];
    }
    __syncthreads();
    const int CH = hd / E, KG = 256 / CH, ch = tid % CH, g = tid / CH;
    const T* vb = vc + ((int64_t)b * Tmax + j0) * d + h * hd + ch * E;
    uint4 vpre[GA_VPRE];
#pragma unroll
    for (int u = 0; u < GA_VPRE; ++u) {
        const int j = g + u * KG;
        vpre[u] = *reinterpret_cast<const uint4*>(vb + (int64_t)min(j, n - 1) * d);
    }
    const T* kb = kc + ((int64_t)b * Tmax + j0) * d + h * hd;
    float mx = -FLT_MAX;
    for (int j = tid; j < n; j += 256) {
        const T* kr = kb + (int64_t)j * d;
        float acc = 0.f;
        // 16-byte loads of the key row (hd and d are multiples of 8 elements)
        for (int c = 0; c < hd; c += E) {
            const uint4 raw = *reinterpret_cast<const uint4*>(kr + c);
            const T* kv = reinterpret_cast<const T*>(&raw);
#pragma unroll
            for (int e = 0; e < E; ++e) acc += qs[c + e] * to_f32(kv[e]);
        }
        const float v = acc * scale;
        sc[j] = v;
        mx = fmaxf(mx, v);
    }
    mx = block_max_f<256>(mx, rsh);
    float sum = 0.f;
    for (int j = tid; j < n; j += 256) {
        const float e = __expf(sc[j] - mx);
        sc[j] = e;
        sum += e;
    }
    sum = block_sum_f<256>(sum, rsh);   // its barriers also order the weight writes before the reads below
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < GA_VPRE; ++u) {
        const int j = g + u * KG;
        if (j < n) {
            const float p = sc[j];
            const T* vv = reinterpret_cast<const T*>(&vpre[u]);
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += p * to_f32(vv[e]);
        }
    }
    for (int j = g + GA_VPRE * KG; j < n; j += KG) {
        const uint4 raw = *reinterpret_cast<const uint4*>(vb + (int64_t)j * d);
        const T* vv = reinterpret_cast<const T*>(&raw);
        const float p = sc[j];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += p * to_f32(vv[e]);
    }
    __syncthreads();   // every weight read before the partial rows overwrite sc
    float* red = sc;   // [KG][hd]
#pragma unroll
    for (int e = 0; e < E; ++e) red[g * hd + ch * E + e] = acc[e];
    __syncthreads();
    if (tid < hd) {
        float a = 0.f;
        for (int gg = 0; gg < KG; ++gg) a += red[gg * hd + tid];
        out[(int64_t)b * d + h * hd + tid] = from_f32<T>(a / sum);
    }
}

void gen_attention(bool bf, const void* q, int64_t ldq, const void* knew, int64_t ldk, const void* vnew, int64_t ldv,
                   void* kc, void* vc, void* out, int B, int H, int hd, int pos, int Tmax, int window, hipStream_t s) {
    // the scores, or the partial output rows (256 threads x one 16-byte chunk of floats each)
    const size_t lds = sizeof(float) * (size_t)(pos + 1 > 256 * (bf ? 8 : 4) ? pos + 1 : 256 * (bf ? 8 : 4));
    const float scale = 1.0f / sqrtf((float)hd);
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void*)gen_attention_kernel<bf16>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 4 * 32768);
        (void)hipFuncSetAttribute((const void*)gen_attention_kernel<float>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 4 * 32768);
        attr = true;
    }
    if (bf)
        gen_attention_kernel<bf16><<<B * H, 256, lds, s>>>((const bf16*)q, ldq, (const bf16*)knew, ldk,
                                                           (const bf16*)vnew, ldv, (bf16*)kc, (bf16*)vc, (bf16*)out, H,
                                                           hd, pos, Tmax, window, scale);
    else
        gen_attention_kernel<float><<<B * H, 256, lds, s>>>((const float*)q, ldq, (const float*)knew, ldk,
                                                            (const float*)vnew, ldv, (float*)kc, (float*)vc,
                                                            (float*)out, H, hd, pos, Tmax, window, scale);
}

// ---------------------------------------------------------------- one draw per sequence

// One workgroup of 1024 threads per sequence. Passes that need no order read
// the row with strided, coalesced accesses; the passes that walk it in token
// order use contiguous ranges (thread t owns [t C, (t + 1) C), C =
// ceil(Vp / 1024), so thread order is token order). Steps: softcap in place
// (and the copy out); the maximum; greedy for temperature 0 (first index of
// the maximum); for 0 < top_k < Vp the k-th largest value by a radix select
// over the order-preserving keys (four passes of 256-bin histograms in LDS,
// most significant byte first), keeping every larger value and the
// lowest-index ties; weights exp((z - max) / T) summed per thread in token
// order and scanned across threads; the draw is the first token whose
// running sum exceeds u * total, u from Philox4x64-10 at counter (step,
// sequence) with key (seed, sampling stream).
// Each histogram bin has GS_SUB copies (lane % GS_SUB picks one): the logits
// of a row share their leading key bytes, so with one counter per bin the
// first passes would send nearly every increment to the same LDS word. The
// bin holding the k-th largest key comes from a scan of the bin totals in
// descending bin order.
constexpr int GS_THREADS = 1024;
constexpr int GS_SUB = 32;

__global__ __launch_bounds__(GS_THREADS) void gen_sample_kernel(float* logits, int Vp, float cap, float temperature,
                                                                int top_k, uint64_t seed, int step, int32_t* seq,
                                                                int64_t ld_seq, int pos_out, float* logits_out) {
    __shared__ float fsh[GS_THREADS / 64 + 1];
    __shared__ int ish[GS_THREADS / 64 + 1];
    __shared__ int hist[256 * GS_SUB];   // [bin][copy]
    __shared__ uint32_t sel[2];         // selected prefix, count still needed
    const int b = blockIdx.x, tid = threadIdx.x;
    float* z = logits + (int64_t)b * Vp;
    float mx = -FLT_MAX;
    for (int i = tid; i < Vp; i += GS_THREADS) {
        float v = z[i];
        if (cap > 0.f) {
            v = cap * tanhf(v / cap);
            z[i] = v;
        }
        if (logits_out) logits_out[(int64_t)b * Vp + i] = v;
        mx = fmaxf(mx, v);
    }
    mx = block_max_f<GS_THREADS>(mx, fsh);   // its barriers order the softcap writes before the reads below
    const int chunk = ceil_div(Vp, GS_THREADS);
    const int i0 = min(Vp, tid * chunk), i1 = min(Vp, i0 + chunk);
    int32_t* dst = seq + (int64_t)b * ld_seq + pos_out;
    if (temperature == 0.f) {
        int first = INT_MAX;
        for (int i = i0; i < i1; ++i)
            if (z[i] == mx) { first = i; break; }
        first = -block_max_i<GS_THREADS>(-first, ish);
        if (tid == 0) *dst = first;
        return;
    }
    const bool trunc = top_k > 0 && top_k < Vp;
    uint32_t thr = 0;
    int need = 0, tie_before = 0;
    if (trunc) {
        // radix select of the k-th largest key, most significant byte first
        if (tid == 0) { sel[0] = 0; sel[1] = (uint32_t)top_k; }
        const int sub = tid & (GS_SUB - 1);
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            const uint32_t hmask = pass ? (0xFFFFFFFFu << (32 - 8 * pass)) : 0u;
            for (int i = tid; i < 256 * GS_SUB; i += GS_THREADS) hist[i] = 0;
            __syncthreads();
            const uint32_t prefix = sel[0], rem = sel[1];
            for (int i = tid; i < Vp; i += GS_THREADS) {
                const uint32_t k = order_key(z[i]);
                if ((k & hmask) == prefix) atomicAdd(&hist[((k >> shift) & 255) * GS_SUB + sub], 1);
            }
            __syncthreads();
            // thread t < 256 takes bin 255 - t: its total, and by an exclusive
            // scan the number of keys in higher bins
            int cnt = 0;
            if (tid < 256) {
                const int* hb = hist + (255 - tid) * GS_SUB;
#pragma unroll 8
                for (int u = 0; u < GS_SUB; ++u) cnt += hb[(u + tid) & (GS_SUB - 1)];
            }
            int all = 0;
            const int above = block_excl_scan<GS_THREADS, int>(cnt, ish, &all);
            // the bin where the count of higher keys first reaches rem (bin 0
            // takes what is left); its scan barriers ordered every read of sel
            if (tid < 256 && (uint32_t)above < rem && ((uint32_t)(above + cnt) >= rem || tid == 255)) {
                sel[0] = prefix | ((uint32_t)(255 - tid) << shift);
                sel[1] = rem - (uint32_t)above;
            }
            __syncthreads();
        }
        thr = sel[0];
        int gt = 0, ties = 0;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = order_key(z[i]);
            gt += k > thr;
            ties += k == thr;
        }
        need = top_k - block_sum_i<GS_THREADS>(gt, ish);
        int tot = 0;
        tie_before = block_excl_scan<GS_THREADS, int>(ties, ish, &tot);
    }
    const float inv_t = 1.0f / temperature;
    float s = 0.f;
    int last = -1;
    {
        int tr = tie_before;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = order_key(z[i]);
            const bool keep = !trunc || k > thr || (k == thr && tr++ < need);
            if (keep) {
                s += __expf((z[i] - mx) * inv_t);
                last = i;
            }
        }
    }
    float total = 0.f;
    const float pre = block_excl_scan<GS_THREADS, float>(s, fsh, &total);
    uint64_t c4[4] = {(uint64_t)step, (uint64_t)b, 0, 0};
    gen_philox(c4, seed, SAMPLE_STREAM);
    const double u = ((double)(c4[0] >> 11) + 0.5) * 0x1.0p-53;
    const float target = (float)(u * (double)total);
    // the owner: the last thread with kept weight whose prefix does not exceed the target
    const int owner = block_max_i<GS_THREADS>((last >= 0 && pre <= target) ? tid : -1, ish);
    if (tid == owner) {
        int tr = tie_before, tok = last;
        float run = pre;
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = order_key(z[i]);
            const bool keep = !trunc || k > thr || (k == thr && tr++ < need);
            if (!keep) continue;
            run += __expf((z[i] - mx) * inv_t);
            if (run > target) { tok = i; break; }
        }
        *dst = tok;
    }
}

// Top-k draw (temperature > 0, 0 < top_k <= GS_MAXK, top_k < Vp); the same
// draw as gen_sample_kernel with every pass over the row coalesced (thread t
// visits tokens t, t + 1024, ..., eight loads in flight) and five passes in
// all: the softcap, the maximum and the first radix histogram share one; the
// k-th largest key thr comes from the same radix select, whose last pass
// also gives the count of keys equal to thr and how many of them are kept
// (rem). The kept set (every larger key and the rem lowest-index ties, which
// are ranked with ballots over the strided layout in an extra pass only when
// some ties are dropped) is gathered in LDS, put in token order by counting
// smaller indices, and one thread sums its weights exp((z - max) / T) in
// token order and walks them to the first running sum above u * total.
constexpr int GS_MAXK = 1024;
constexpr int GS_MAXROUND = 64;   // rounds of 1024 tokens: Vp <= 65536
constexpr int GS_BATCH = 8;       // loads in flight per thread and sweep step

__global__ __launch_bounds__(GS_THREADS) void gen_sample_topk_kernel(float* logits, int Vp, float cap,
                                                                     float temperature, int top_k, uint64_t seed,
                                                                     int step, int32_t* seq, int64_t ld_seq,
                                                                     int pos_out, float* logits_out) {
    __shared__ float fsh[GS_THREADS / 64 + 1];
    __shared__ int ish[GS_THREADS / 64 + 1];
    __shared__ int hist[256 * GS_SUB];   // [bin][copy]; later the tie counts and the sorted kept set
    __shared__ uint32_t sel[3];          // selected prefix, keys still needed from it, keys equal to it
    __shared__ int kcount;
    __shared__ int kidx[GS_MAXK];
    __shared__ float kval[GS_MAXK];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    float* z = logits + (int64_t)b * Vp;
    // f(i, z[i]) for every token of this thread, GS_BATCH loads issued together
    auto sweep = [&](auto&& f) {
        for (int base = tid; base < Vp; base += GS_BATCH * GS_THREADS) {
            float v[GS_BATCH];
#pragma unroll
            for (int j = 0; j < GS_BATCH; ++j) v[j] = z[min(base + j * GS_THREADS, Vp - 1)];
#pragma unroll
            for (int j = 0; j < GS_BATCH; ++j)
                if (base + j * GS_THREADS < Vp) f(base + j * GS_THREADS, v[j]);
        }
    };
    const int sub = tid & (GS_SUB - 1);
    for (int i = tid; i < 256 * GS_SUB; i += GS_THREADS) hist[i] = 0;
    if (tid == 0) { sel[0] = 0; sel[1] = (uint32_t)top_k; sel[2] = 0; kcount = 0; }
    __syncthreads();
    // pass 0: softcap in place (and the copy out), the maximum, the histogram of the leading key byte
    float mx = -FLT_MAX;
    sweep([&](int i, float v) {
        if (cap > 0.f) {
            v = cap * tanhf(v / cap);
            z[i] = v;
        }
        if (logits_out) logits_out[(int64_t)b * Vp + i] = v;
        mx = fmaxf(mx, v);
        atomicAdd(&hist[(order_key(v) >> 24) * GS_SUB + sub], 1);
    });
    mx = block_max_f<GS_THREADS>(mx, fsh);   // its barriers order the softcap writes and the histogram
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        const uint32_t prefix = sel[0], rem = sel[1];
        if (pass > 0) {
            const uint32_t hmask = 0xFFFFFFFFu << (32 - 8 * pass);
            for (int i = tid; i < 256 * GS_SUB; i += GS_THREADS) hist[i] = 0;
            __syncthreads();
            sweep([&](int, float v) {
                const uint32_t k = order_key(v);
                if ((k & hmask) == prefix) atomicAdd(&hist[((k >> shift) & 255) * GS_SUB + sub], 1);
            });
            __syncthreads();
        }
        // thread t < 256 takes bin 255 - t: its total, and by an exclusive
        // scan the number of keys in higher bins
        int cnt = 0;
        if (tid < 256) {
            const int* hb = hist + (255 - tid) * GS_SUB;
#pragma unroll 8
            for (int u = 0; u < GS_SUB; ++u) cnt += hb[(u + tid) & (GS_SUB - 1)];
        }
        int all = 0;
        const int above = block_excl_scan<GS_THREADS, int>(cnt, ish, &all);
        // the bin where the count of higher keys first reaches rem (bin 0 takes
        // what is left); the scan's barriers ordered every read of sel
        if (tid < 256 && (uint32_t)above < rem && ((uint32_t)(above + cnt) >= rem || tid == 255)) {
            sel[0] = prefix | ((uint32_t)(255 - tid) << shift);
            sel[1] = rem - (uint32_t)above;
            sel[2] = (uint32_t)cnt;
        }
        __syncthreads();
    }
    const uint32_t thr = sel[0];
    const int need = (int)sel[1], ties = (int)sel[2];   // keys equal to thr: kept, and in all
    auto gather = [&](int i, float v) {
        const int slot = atomicAdd(&kcount, 1);   // exactly top_k slots are taken
        if (slot < GS_MAXK) {
            kidx[slot] = i;
            kval[slot] = v;
        }
    };
    if (ties == need) {
        sweep([&](int i, float v) {
            if (order_key(v) >= thr) gather(i, v);
        });
    } else {
        // ties ranked in token order: per round u (tokens u * 1024 .. + 1023) a
        // ballot per wave; an exclusive scan of the (round, wave) counts gives
        // the ties before each wave's slice
        constexpr int NW = GS_THREADS / 64;
        int* tcnt = hist;   // [GS_MAXROUND][NW]
        const int rounds = ceil_div(Vp, GS_THREADS);
        for (int u = 0; u < rounds; ++u) {
            const int i = u * GS_THREADS + tid;
            const uint64_t tm = __ballot(i < Vp && order_key(z[min(i, Vp - 1)]) == thr);
            if (lane == 0) tcnt[u * NW + w] = __popcll(tm);
        }
        __syncthreads();
        {
            const int n = rounds * NW;   // <= GS_THREADS
            const int v = tid < n ? tcnt[tid] : 0;
            int tot = 0;
            const int ex = block_excl_scan<GS_THREADS, int>(v, ish, &tot);   // its barriers order the read above
            if (tid < n) tcnt[tid] = ex;
        }
        __syncthreads();
        const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
        for (int u = 0; u < rounds; ++u) {
            const int i = u * GS_THREADS + tid;
            const float v = z[min(i, Vp - 1)];
            const uint32_t k = order_key(v);
            const bool tie = i < Vp && k == thr;
            const uint64_t tm = __ballot(tie);
            if (i < Vp && (k > thr || (tie && tcnt[u * NW + w] + __popcll(tm & lt) < need))) gather(i, v);
        }
    }
    __syncthreads();
    // exactly top_k kept: each finds its place in token order
    int* sidx = hist;
    float* sw = reinterpret_cast<float*>(hist + GS_MAXK);
    const float inv_t = 1.0f / temperature;
    if (tid < top_k) {
        const int mine = kidx[tid];
        int rank = 0;
        for (int m = 0; m < top_k; ++m) rank += kidx[m] < mine;
        sidx[rank] = mine;
        sw[rank] = __expf((kval[tid] - mx) * inv_t);
    }
    __syncthreads();
    if (tid == 0) {
        float total = 0.f;
        for (int j = 0; j < top_k; ++j) total += sw[j];
        uint64_t c4[4] = {(uint64_t)step, (uint64_t)b, 0, 0};
        gen_philox(c4, seed, SAMPLE_STREAM);
        const double uu = ((double)(c4[0] >> 11) + 0.5) * 0x1.0p-53;
        const float target = (float)(uu * (double)total);
        int tok = sidx[top_k - 1];
        float run = 0.f;
        for (int j = 0; j < top_k; ++j) {
            run += sw[j];
            if (run > target) { tok = sidx[j]; break; }
        }
        seq[(int64_t)b * ld_seq + pos_out] = tok;
    }
}

void gen_sample(float* logits, int B, int Vp, float cap, float temperature, int top_k, uint64_t seed, int step,
                int32_t* seq, int64_t ld_seq, int pos_out, float* logits_out, hipStream_t s) {
    if (temperature > 0.f && top_k > 0 && top_k <= GS_MAXK && top_k < Vp && Vp <= GS_THREADS * GS_MAXROUND)
        gen_sample_topk_kernel<<<B, GS_THREADS, 0, s>>>(logits, Vp, cap, temperature, top_k, seed, step, seq, ld_seq,
                                                         pos_out, logits_out);
    else
        gen_sample_kernel<<<B, GS_THREADS, 0, s>>>(logits, Vp, cap, temperature, top_k, seed, step, seq, ld_seq,
                                                    pos_out, logits_out);
}

// ---------------------------------------------------------------- products at decode shapes

// C[m, n] = epilogue(sum_k A[m, k] W[n, k]) for m < M <= 16, bf16 A [M, K]
// (row stride lda) and W [N, K] (row stride ldb), K % 32 == 0. The 16 rows of
// A (rows past M read as zero) sit in LDS; each workgroup owns 16 consecutive
// columns and its eight waves split K; a wave loads 16 bytes of each of the 16
// weight rows per 32-deep step (lane l: row l % 16, k 8 (l / 16) .. + 7; the A
// fragment the same) into v_mfma_f32_16x16x32_bf16, and the partial 16 x 16
// tiles (lane l: column l % 16, rows 4 (l / 16) .. + 3) are summed in wave
// order before the epilogue. Decode steps read every weight once, so the loop
// is unrolled to keep several loads per lane in flight.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int SK_WAVES = 8;
constexpr int SK_LNV = 3;      // float4 per lane of a normalised row kept in registers: K <= 768
constexpr int SK_ABATCH = 6;   // 16-byte activation pieces loaded together per thread
constexpr int SK_SPLIT_WIDE = 2;   // waves splitting K per column group of a wide product

// CG groups of 16 columns per workgroup (CG = 1: all eight waves split K; CG
// = 4, for wide products such as the head: two waves per group, so the
// staged activations serve 64 columns)
template <int EPI, typename TC, bool LN, int CG>
__global__ __launch_bounds__(64 * SK_WAVES) void skinny_gemm_kernel(Gemm g) {
    extern __shared__ __attribute__((aligned(16))) bf16 As[];   // [16][K + 8]
    __shared__ f32x4_t part[SK_WAVES][64];
    constexpr int KW = SK_WAVES / CG;   // waves splitting K in a column group
    const int K = g.K, ldl = K + 8;
    const bf16* W = (const bf16*)g.B;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, cg = w / KW, kw = w % KW;
    const int n0 = (blockIdx.x * CG + cg) * 16;
    const int r = lane & 15, kq = lane >> 4;
    const int nrow = min(n0 + r, g.N - 1);   // columns past N feed only unstored outputs
    // wave kw of a group takes the k range [kw K / KW, (kw + 1) K / KW) rounded
    // to 32-deep steps; its weight fragments are loaded first, so that their
    // latency overlaps the staging (or LayerNorm) of the activations below
    const int nst = K / 32, s0 = kw * nst / KW, s1 = (kw + 1) * nst / KW;
    const bf16* wr = W + (int64_t)nrow * g.ldb + 8 * kq;
    constexpr int MAXST = 4096 / 32 / SK_WAVES;   // steps per wave: K <= 4096 / CG
    static_assert(MAXST * 32 * KW == 4096 / CG, "weight steps per wave");
    bf16x8_t wv[MAXST];
#pragma unroll
    for (int i = 0; i < MAXST; ++i)
        if (s0 + i < s1) wv[i] = *reinterpret_cast<const bf16x8_t*>(wr + 32 * (s0 + i));
    // the epilogue's own operands (bias, residual) are loaded by the storing
    // wave now, so their latency overlaps the products
    constexpr bool HAS_BIAS = EPI == EPI_BIAS || EPI == EPI_BIAS_ACT || EPI == EPI_BIAS_RESID;
    float bias_n = 0.f, res[4] = {0.f, 0.f, 0.f, 0.f};
    if (kw == 0 && n0 + r < g.N) {
        if constexpr (HAS_BIAS) bias_n = g.bias[n0 + r];
        if constexpr (EPI == EPI_BIAS_RESID) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (4 * kq + i < g.M) res[i] = g.resid[(int64_t)(4 * kq + i) * g.ldc + n0 + r];
        }
    }
    if constexpr (LN) {
        // wave w normalises rows w, w + SK_WAVES: the LayerNorm kernel's
        // arithmetic in its order (lane sums over float4 chunks, wave sums,
        // biased variance, rsqrt), stored as bf16
        const int r0 = w, r1 = w + SK_WAVES;
        if (K <= 256 * SK_LNV) {
            // the rows, gains and biases loaded once, together
            float4 xv[2][SK_LNV], gv[SK_LNV], bv[SK_LNV];
            const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < SK_LNV; ++j) {
                const int c = 4 * lane + 256 * j;
                gv[j] = c < K ? load4(g.ln_g + c) : z4;
                bv[j] = c < K ? load4(g.ln_b + c) : z4;
                xv[0][j] = c < K && r0 < g.M ? load4((const float*)g.A + (int64_t)r0 * g.lda + c) : z4;
                xv[1][j] = c < K && r1 < g.M ? load4((const float*)g.A + (int64_t)r1 * g.lda + c) : z4;
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int rr = q ? r1 : r0;
                bf16* dst = As + rr * ldl;
                if (rr < g.M) {
                    float sum = 0.f;
#pragma unroll
                    for (int j = 0; j < SK_LNV; ++j)
                        if (4 * lane + 256 * j < K) sum += (xv[q][j].x + xv[q][j].y) + (xv[q][j].z + xv[q][j].w);
                    const float mu = wave_sum(sum) / K;
                    float s2 = 0.f;
#pragma unroll
                    for (int j = 0; j < SK_LNV; ++j)
                        if (4 * lane + 256 * j < K) {
                            const float4 v = xv[q][j];
                            const float a = v.x - mu, b = v.y - mu, cc = v.z - mu, dd = v.w - mu;
                            s2 += (a * a + b * b) + (cc * cc + dd * dd);
                        }
                    const float rs = 1.0f / sqrtf(wave_sum(s2) / K + g.ln_eps);
#pragma unroll
                    for (int j = 0; j < SK_LNV; ++j) {
                        const int c = 4 * lane + 256 * j;
                        if (c < K) {
                            const float4 v = xv[q][j], gg = gv[j], bb = bv[j];
                            float4 o;
                            o.x = (v.x - mu) * rs * gg.x + bb.x;
                            o.y = (v.y - mu) * rs * gg.y + bb.y;
                            o.z = (v.z - mu) * rs * gg.z + bb.z;
                            o.w = (v.w - mu) * rs * gg.w + bb.w;
                            store4(dst + c, o);
                        }
                    }
                } else {
                    for (int c = 4 * lane; c < K; c += 256) store4(dst + c, z4);
                }
            }
        } else {
            for (int r = w; r < 16; r += SK_WAVES) {
                bf16* dst = As + r * ldl;
                if (r < g.M) {
                    const float* xr = (const float*)g.A + (int64_t)r * g.lda;
                    float sum = 0.f;
                    for (int c = 4 * lane; c < K; c += 256) {
                        const float4 v = load4(xr + c);
                        sum += (v.x + v.y) + (v.z + v.w);
                    }
                    const float mu = wave_sum(sum) / K;
                    float s2 = 0.f;
                    for (int c = 4 * lane; c < K; c += 256) {
                        const float4 v = load4(xr + c);
                        const float a = v.x - mu, b = v.y - mu, cc = v.z - mu, dd = v.w - mu;
                        s2 += (a * a + b * b) + (cc * cc + dd * dd);
                    }
                    const float rs = 1.0f / sqrtf(wave_sum(s2) / K + g.ln_eps);
                    for (int c = 4 * lane; c < K; c += 256) {
                        const float4 v = load4(xr + c), gg = load4(g.ln_g + c), bb = load4(g.ln_b + c);
                        float4 o;
                        o.x = (v.x - mu) * rs * gg.x + bb.x;
                        o.y = (v.y - mu) * rs * gg.y + bb.y;
                        o.z = (v.z - mu) * rs * gg.z + bb.z;
                        o.w = (v.w - mu) * rs * gg.w + bb.w;
                        store4(dst + c, o);
                    }
                } else {
                    for (int c = 4 * lane; c < K; c += 256) store4(dst + c, make_float4(0.f, 0.f, 0.f, 0.f));
                }
            }
        }
    } else {
        // the 16-byte pieces of the 16 rows in batches of SK_ABATCH per
        // thread, each batch loaded before its first piece is stored (one
        // batch covers K <= 1536)
        const bf16* A = (const bf16*)g.A;
        const int nch = 16 * (K / 8);
        for (int i0 = threadIdx.x; i0 < nch; i0 += SK_ABATCH * 64 * SK_WAVES) {
            bf16x8_t av[SK_ABATCH];
#pragma unroll
            for (int u = 0; u < SK_ABATCH; ++u) {
                const int i = i0 + u * 64 * SK_WAVES;
                const int r = i / (K / 8), c = (i % (K / 8)) * 8;
                bf16x8_t v = {};
                if (i < nch && r < g.M) v = *reinterpret_cast<const bf16x8_t*>(A + (int64_t)r * g.lda + c);
                av[u] = v;
            }
#pragma unroll
            for (int u = 0; u < SK_ABATCH; ++u) {
                const int i = i0 + u * 64 * SK_WAVES;
                const int r = i / (K / 8), c = (i % (K / 8)) * 8;
                if (i < nch) *reinterpret_cast<bf16x8_t*>(As + r * ldl + c) = av[u];
            }
        }
    }
    __syncthreads();
    const bf16* ar = As + r * ldl + 8 * kq;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MAXST; ++i)
        if (s0 + i < s1) {
            const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(ar + 32 * (s0 + i));
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, wv[i], acc, 0, 0, 0);
        }
    part[w][lane] = acc;
    __syncthreads();
    if (kw == 0) {
        // the group's partial tiles, summed in wave order
        f32x4_t t = part[w][lane];
#pragma unroll
        for (int v = 1; v < KW; ++v) t += part[w + v][lane];
        const int n = n0 + r;
        if (n < g.N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * kq + i;
                if (m >= g.M) continue;
                // the arithmetic of epilogue_store, with the preloaded operands
                const int64_t o = (int64_t)m * g.ldc + n;
                if constexpr (EPI == EPI_BIAS_RESID) {
                    ((float*)g.C)[o] = res[i] + (t[i] + bias_n);
                } else if constexpr (EPI == EPI_BIAS) {
                    ((TC*)g.C)[o] = from_f32<TC>(t[i] + bias_n);
                } else if constexpr (EPI == EPI_BIAS_ACT) {
                    float a, da;
                    act_and_grad_rt(g.act, t[i] + bias_n, a, da);
                    ((TC*)g.C)[o] = from_f32<TC>(da);
                    ((TC*)g.C2)[o] = from_f32<TC>(a);
                } else {
                    epilogue_store<TC, EPI>(g, m, n, t[i]);
                }
            }
        }
    }
}

bool skinny_gemm_ok(const Gemm& g) {
    const bool a_ok = g.ln_g ? (g.K % 4 == 0 && ((uintptr_t)g.A & 15) == 0 && g.lda % 4 == 0 && g.ln_b)
                             : (g.lda % 8 == 0 && ((uintptr_t)g.A & 15) == 0);
    return g.in_bf && g.a_kc && g.b_kc && g.M >= 1 && g.M <= 16 && g.K % 32 == 0 && g.K <= 4096 && a_ok &&
           g.ldb % 8 == 0 && ((uintptr_t)g.B & 15) == 0;
}

template <int EPI, typename TC, int CG>
static void skinny_launch_cg(const Gemm& g, size_t lds, hipStream_t s) {
    static bool attr = false;
    if (!attr) {
        const int mx = (int)(sizeof(bf16) * 16 * (4096 + 8));
        (void)hipFuncSetAttribute((const void*)skinny_gemm_kernel<EPI, TC, false, CG>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, mx);
        (void)hipFuncSetAttribute((const void*)skinny_gemm_kernel<EPI, TC, true, CG>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, mx);
        attr = true;
    }
    const unsigned grid = (unsigned)ceil_div(g.N, 16 * CG);
    if (g.ln_g) skinny_gemm_kernel<EPI, TC, true, CG><<<grid, 64 * SK_WAVES, lds, s>>>(g);
    else skinny_gemm_kernel<EPI, TC, false, CG><<<grid, 64 * SK_WAVES, lds, s>>>(g);
}

// wide products (the head) stage the activations once per 64 columns; a
// wave holds at most MAXST 32-deep steps of weights, so with CG groups K <= 4096 / CG
template <int EPI, typename TC>
static void skinny_launch(const Gemm& g, unsigned, size_t lds, hipStream_t s) {
    constexpr int CGW = SK_WAVES / SK_SPLIT_WIDE;
    if (g.N >= 4096 && g.K <= 4096 / CGW) skinny_launch_cg<EPI, TC, CGW>(g, lds, s);
    else skinny_launch_cg<EPI, TC, 1>(g, lds, s);
}

void skinny_gemm(const Gemm& g, hipStream_t s) {
    const unsigned grid = (unsigned)ceil_div(g.N, 16);
    const size_t lds = sizeof(bf16) * 16 * (size_t)(g.K + 8);
    switch (g.epi) {
        case EPI_STORE:
            if (g.c_bf) skinny_launch<EPI_STORE, bf16>(g, grid, lds, s);
            else skinny_launch<EPI_STORE, float>(g, grid, lds, s);
            break;
        case EPI_BIAS: skinny_launch<EPI_BIAS, bf16>(g, grid, lds, s); break;
        case EPI_BIAS_ACT: skinny_launch<EPI_BIAS_ACT, bf16>(g, grid, lds, s); break;
        case EPI_BIAS_RESID: skinny_launch<EPI_BIAS_RESID, float>(g, grid, lds, s); break;
        default: break;
    }
}

}  // namespace gk
