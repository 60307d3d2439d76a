// Dispatch of the bf16 matrix-core GEMM (kernel in gemm_mfma_kernel.h):
// configuration and split-K choice, launch per operand layout, and the
// deterministic sum of split-K slices.
#include "gemm_mfma_kernel.h"

#include <algorithm>
#include <cstdio>
#include <vector>

namespace gk {

// Sums the split-K slices in a fixed order (deterministic) and applies the
// epilogue; one thread per 8 consecutive outputs of a row.
template <int EPI, int OUTBF, int ACT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(Gemm g, const float* part, int splits) {
    using TC = typename std::conditional<OUTBF != 0, bf16, float>::type;
    const int cpr = g.N / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)g.M * cpr) return;
    const int row = (int)(idx / cpr), col = 8 * (int)(idx % cpr);
    const int64_t mn = (int64_t)g.M * g.N, o = (int64_t)row * g.N + col;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    for (int z = 0; z < splits; ++z) {
        const float4 x = *reinterpret_cast<const float4*>(part + z * mn + o);
        const float4 y = *reinterpret_cast<const float4*>(part + z * mn + o + 4);
        a.x += x.x; a.y += x.y; a.z += x.z; a.w += x.w;
        b.x += y.x; b.y += y.y; b.z += y.z; b.w += y.w;
    }
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float bv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) bv[e] = 0.f;
    if constexpr (EPI == EPI_BIAS || EPI == EPI_BIAS_ACT || EPI == EPI_BIAS_RESID) {
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[e] = g.bias[col + e];
    }
    epilogue_chunk8<TC, EPI, ACT>(g, row, col, v, bv);
}

// Override of the automatic choice through the test entry point
// (gemm_mfma_force; cfg index as in GemmCfg, splits 0 = automatic).
static int g_force_cfg = -1, g_force_splits = 0;
void gemm_mfma_force(int cfg, int splits) {
    g_force_cfg = cfg >= 0 && cfg < CFG_COUNT ? cfg : -1;
    g_force_splits = splits;
}
int gemm_mfma_num_configs() { return CFG_COUNT; }
static bool forced(int* cfg, int* splits) {
    if (g_force_cfg < 0) return false;
    *cfg = g_force_cfg;
    *splits = g_force_splits;
    return true;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

bool gemm_mfma_ok(const Gemm& g) {
    if (!g.in_bf || g.K % 32) return false;
    if (!aligned16(g.A) || !aligned16(g.B)) return false;
    if (g.lda % 8 || g.ldb % 8) return false;
    if (!g.a_kc && (g.M % 8 || g.M < 8)) return false;
    if (g.N % 8 || g.N < 8 || g.ldc % 8) return false;     // 16-byte epilogue chunks
    if (!g.a_kc && g.b_kc) return false;     // orientation not used by the training step
    if (!layout_has_epi(g.a_kc, g.b_kc, g.epi)) return false;   // not instantiated for this layout
    if (g.batch > 1 && (g.epi != EPI_STORE || g.sa % 8 || g.sb % 8 || g.sc % 8 || g.batch > 65535)) return false;
    const bool bias = g.epi == EPI_BIAS || g.epi == EPI_BIAS_ACT || g.epi == EPI_BIAS_RESID;
    if (!aligned16(g.C) || (g.epi == EPI_BIAS_ACT && !aligned16(g.C2)) || (bias && !aligned16(g.bias)) ||
        (g.epi == EPI_BIAS_RESID && !aligned16(g.resid)) || (g.epi == EPI_ACT_GRAD && !aligned16(g.aux)))
        return false;
    return true;
}

static int num_cus() {
    static int n = 0;
    if (!n) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
    }
    return n;
}

// Tile configuration and split-K factor from a cost model: the workgroups
// are spread evenly over the CUs; a CU runs its share at the configuration's
// measured per-CU rate (a lone workgroup of a two-per-CU configuration at
// 60% of it), each workgroup adds its epilogue (fused activations cost more;
// two workgroups per CU overlap it with the other's products), each round of
// workgroup slots a fixed prologue, and split-K its fp32 partials.
// Measured best choices for the products of the 124M-parameter shapes
// (d = 768, F = 3072, Vp = 50304, 16384 rows per micro-batch); other shapes
// use the cost model below.
struct Tuned { int M, N, K; bool a_kc, b_kc; int cfg, splits; };
static const Tuned tuned[] = {
    // forward: X W^T
    {16384, 2304, 768, true, true, CFG_256_192_K64VW8, 1}, {16384, 768, 768, true, true, CFG_128_192_K64, 1},
    {16384, 3072, 768, true, true, CFG_256_256_K64VW8, 1}, {16384, 768, 3072, true, true, CFG_128_192_K64, 1},
    {16384, 50304, 768, true, true, CFG_256_256_K64VW8, 1},
    // input gradients: dY W
    {16384, 3072, 768, true, false, CFG_256_256_K64VW8, 1}, {16384, 768, 3072, true, false, CFG_256_192_K64VW8, 1},
    {16384, 768, 768, true, false, CFG_256_192_K64VW8, 1}, {16384, 768, 2304, true, false, CFG_256_192_K64VW8, 1},
    {16384, 768, 50304, true, false, CFG_256_256_K64VW8, 1},
    // weight gradients: dY^T X
    {768, 3072, 16384, false, false, CFG_256_256_K64VW8, 4}, {3072, 768, 16384, false, false, CFG_256_256_K64VW8, 4},
    {768, 768, 16384, false, false, CFG_128_128_K64R, 8}, {2304, 768, 16384, false, false, CFG_256_256_K64VW8, 8},
    {50304, 768, 16384, false, false, CFG_256_256_K64VW8, 1},
};

// Per-shape overrides of the tuned table (test control, for measurements).
static std::vector<Tuned> g_tune_override;
int gemm_mfma_tune(int M, int N, int K, bool a_kc, bool b_kc, int cfg, int splits) {
    if (cfg < -1 || cfg >= CFG_COUNT || splits < 0) return -1;
    g_tune_override.erase(std::remove_if(g_tune_override.begin(), g_tune_override.end(), [&](const Tuned& e) {
                              return e.M == M && e.N == N && e.K == K && e.a_kc == a_kc && e.b_kc == b_kc;
                          }), g_tune_override.end());
    if (cfg >= 0) g_tune_override.push_back({M, N, K, a_kc, b_kc, cfg, splits > 0 ? splits : 1});
    return 0;
}

GemmPlan gemm_mfma_plan(const Gemm& g, size_t nscratch) {
    struct Cand { int cfg; double rate; };
    static const Cand cands[] = {{CFG_256_128, 3.3e12}, {CFG_128_128, 2.8e12}, {CFG_256_256_K64, 3.5e12},
                                 {CFG_256_192_K64, 3.36e12}, {CFG_128_192_K64, 3.8e12}, {CFG_128_128_K64, 3.3e12}};
    static const int split_opts[] = {1, 2, 3, 4, 6, 8, 12, 16};
    const int64_t mn = (int64_t)g.M * g.N;
    const double out_bytes = out_bf(g) ? 2.0 : 4.0;
    const double epi_s = (g.epi == EPI_BIAS_ACT || g.epi == EPI_ACT_GRAD) ? 0.09e-9 : 0.015e-9;   // per element
    const int cus = num_cus();
    int fcfg = -1, fsplits = 0;
    bool force = forced(&fcfg, &fsplits);
    if (!force)
        for (const Tuned& e : g_tune_override)
            if (!force && e.M == g.M && e.N == g.N && e.K == g.K && e.a_kc == g.a_kc && e.b_kc == g.b_kc) {
                int sp = e.splits;
                while (sp > 1 && (size_t)sp * mn > nscratch) --sp;
                force = true;
                fcfg = e.cfg;
                fsplits = sp;
            }
    if (!force)
        for (const Tuned& e : tuned)
            if (e.M == g.M && e.N == g.N && e.K == g.K && e.a_kc == g.a_kc && e.b_kc == g.b_kc) {
                int sp = e.splits;
                while (sp > 1 && (size_t)sp * mn > nscratch) --sp;
                force = true;
                fcfg = e.cfg;
                fsplits = sp;
                break;
            }
    double best = 1e30;
    int bcfg = CFG_128_128, bsplits = 1;
    for (int ci = 0; ci < CFG_COUNT; ++ci) {
        double rate = 0.0;
        for (const Cand& c : cands)
            if (c.cfg == ci) rate = c.rate;
        if (force ? ci != fcfg : rate == 0.0) continue;
        if (rate == 0.0) rate = 3.0e12;   // forced configuration outside the candidate list
        if (g.K % cfg_bk[ci]) continue;
        const int bm = cfg_bm[ci], bn = cfg_bn[ci], occ = cfg_occ[ci];
        for (int sp : split_opts) {
            if (force && fsplits > 0 && sp != fsplits) continue;
            const int kps = ceil_div(ceil_div(g.K, sp), cfg_bk[ci]) * cfg_bk[ci];
            const int used = ceil_div(g.K, kps);
            if (used != sp) continue;
            if (sp > 1 && ((size_t)sp * mn > nscratch || kps < 256 || g.batch > 1)) continue;
            const int64_t wgs = (int64_t)ceil_div(g.M, bm) * ceil_div(g.N, bn) * sp * std::max(1, g.batch);
            const int64_t per_cu = (wgs + cus - 1) / cus, rounds = (wgs + (int64_t)cus * occ - 1) / ((int64_t)cus * occ);
            // with two workgroups per CU the rate holds for pairs; a workgroup
            // alone on its CU reaches about 60% of it
            const int64_t lone = occ == 2 ? per_cu % 2 : 0;
            double t = ((per_cu - lone) + lone / 0.6) * (2.0 * bm * bn * kps / rate) + per_cu * epi_s * bm * bn / occ +
                       rounds * 2e-6;
            if (sp > 1) t += (2.0 * sp * mn * 4.0 + mn * out_bytes) / 4e12;
            if (t < best) { best = t; bcfg = ci; bsplits = sp; }
        }
    }
    if (force && best == 1e30) {   // the forced configuration or split is outside the model's options
        bcfg = g.K % cfg_bk[fcfg] ? CFG_256_256 : fcfg;
        bsplits = fsplits > 0 ? fsplits : 1;
        while (bsplits > 1 && ((size_t)bsplits * mn > nscratch || g.K / bsplits < 256)) --bsplits;
    }
    // copies through registers address the operands with 32-bit byte offsets
    if (cfg_pipe[bcfg] == 2) {
        auto span = [](bool kc, int rows, int k, int64_t ld) {
            return 2 * (kc ? (int64_t)(rows - 1) * ld + k : (int64_t)(k - 1) * ld + rows);
        };
        if (span(g.a_kc, g.M, g.K, g.lda) >= ((int64_t)1 << 31) || span(g.b_kc, g.N, g.K, g.ldb) >= ((int64_t)1 << 31)) {
            switch (bcfg) {
                case CFG_256_256_K64VW8: bcfg = CFG_256_256_K64RW8; break;
                case CFG_256_192_K64VW8: bcfg = CFG_256_192_K64RW8; break;
                default: bcfg = CFG_128_128_K64R; break;
            }
        }
    }
    if (g.batch > 1) bsplits = 1;   // batched products run every entry over the whole K
    GemmPlan p{};
    p.cfg = bcfg;
    p.splits = bsplits;
    p.bm = (bsplits == 1 && g.epi == EPI_ACT_GRAD) ? cfg_bm[bcfg] : 0;
    const bool relu = bsplits == 1 && (g.epi == EPI_BIAS_ACT || g.epi == EPI_ACT_GRAD) && g.act == ACT_RELU2;
    snprintf(p.name, sizeof(p.name), "gemm_mfma_kernel<%d, %d, %d, %d, %d, %d, %d, %d, %s, %s, %d, %d, %d, %s>",
             cfg_bm[bcfg], cfg_bn[bcfg], cfg_bk[bcfg], cfg_ns[bcfg], cfg_occ[bcfg], cfg_pipe[bcfg],
             cfg_wgm[bcfg], cfg_wgn[bcfg], g.a_kc ? "true" : "false", g.b_kc ? "true" : "false",
             bsplits > 1 ? 0 : g.epi, bsplits > 1 ? 0 : out_bf(g), relu ? 1 : 0, bsplits > 1 ? "true" : "false");
    return p;
}

void gemm_mfma_main(const Gemm& g, const GemmPlan& p, float* scratch, hipStream_t s) {
    if (g.a_kc && g.b_kc) gemm_mfma_run_kk(g, p, scratch, s);
    else if (g.a_kc) gemm_mfma_run_kc(g, p, scratch, s);
    else gemm_mfma_run_cc(g, p, scratch, s);
}

void gemm_mfma_reduce(const Gemm& g, const GemmPlan& p, const float* scratch, hipStream_t s) {
    if (p.splits <= 1) return;
    const int64_t chunks = (int64_t)g.M * (g.N / 8);
    const unsigned nb = (unsigned)((chunks + 255) / 256);
    const bool relu = g.act == ACT_RELU2;
    switch (g.epi) {
        case EPI_STORE:
            if (g.c_bf) splitk_reduce_kernel<EPI_STORE, 1, 0><<<nb, 256, 0, s>>>(g, scratch, p.splits);
            else splitk_reduce_kernel<EPI_STORE, 0, 0><<<nb, 256, 0, s>>>(g, scratch, p.splits);
            break;
        case EPI_BIAS: splitk_reduce_kernel<EPI_BIAS, 1, 0><<<nb, 256, 0, s>>>(g, scratch, p.splits); break;
        case EPI_BIAS_ACT:
            if (relu) splitk_reduce_kernel<EPI_BIAS_ACT, 1, ACT_RELU2><<<nb, 256, 0, s>>>(g, scratch, p.splits);
            else splitk_reduce_kernel<EPI_BIAS_ACT, 1, ACT_GELU><<<nb, 256, 0, s>>>(g, scratch, p.splits);
            break;
        case EPI_BIAS_RESID: splitk_reduce_kernel<EPI_BIAS_RESID, 0, 0><<<nb, 256, 0, s>>>(g, scratch, p.splits); break;
        case EPI_ACT_GRAD:
            if (relu) splitk_reduce_kernel<EPI_ACT_GRAD, 1, ACT_RELU2><<<nb, 256, 0, s>>>(g, scratch, p.splits);
            else splitk_reduce_kernel<EPI_ACT_GRAD, 1, ACT_GELU><<<nb, 256, 0, s>>>(g, scratch, p.splits);
            break;
        case EPI_ACCUM: splitk_reduce_kernel<EPI_ACCUM, 0, 0><<<nb, 256, 0, s>>>(g, scratch, p.splits); break;
    }
}

void gemm_f8(int M, int N, int K, const void* A8, int64_t lda, const void* B8, int64_t ldb, void* C, int64_t ldc,
             const float* inv_sa_sb, hipStream_t s) {
    Gemm g{};
    g.M = M; g.N = N; g.K = K / 2;           // the kernel counts 2-byte units
    g.A = A8; g.lda = lda / 2; g.a_kc = true;
    g.B = B8; g.ldb = ldb / 2; g.b_kc = true;
    g.C = C; g.ldc = ldc; g.c_bf = true;
    g.epi = EPI_STORE;
    g.in_bf = true;
    g.out_scale = inv_sa_sb;
    gemm_mfma_run_f8(g, s);
}

}  // namespace gk
