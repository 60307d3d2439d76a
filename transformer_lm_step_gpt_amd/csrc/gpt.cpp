// Host engine and C ABI of the GPT-2 training-step library (see include/gpt.h).
//
// Owns: the parameter table, the carving of the caller's workspace, the
// per-micro-step launch schedule (forward, fused cross-entropy, backward),
// gradient accumulation with a lazy zero, the clip + AdamW update, error
// state and optional per-kernel-class event timing.
//
// Training step: "NanoGPT Speedrun baseline" (cruxr.ai), "Configuración del
// Entrenamiento"; "Zero to Hero, lecture 9: reproducing GPT-2 (124M)"
// (ai.flicky.cc), "Раздел 1 / Архитектура", "Связанные веса и
// инициализация", "Оптимизатор, клиппинг, расписание", "Накопление
// градиентов".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gpt.h"
#include "../../include/gpt_testing.h"
#include "host_model.h"
#include "kernels.h"

namespace {

using gpth::LayerIdx;
using gpth::Table;
using gpth::TensorInfo;
using gpth::build_table;
using gpth::INIT_NORMAL;
using gpth::INIT_PROJ;
using gpth::INIT_ZERO;
using gpth::INIT_ONE;

// ---------------------------------------------------------------- workspace layout

struct Ws {
    float *params = nullptr, *grads = nullptr, *m = nullptr, *v = nullptr;
    void* wbf = nullptr;
    std::vector<float*> x_in, x_mid;
    float* x_fin = nullptr;
    float *ln_mean = nullptr, *ln_rstd = nullptr;
    // per layer: LN outputs, qkv, normalised/rotated q,k, attention output, the MLP
    // activation's derivative at its input (for the backward product) and the activation
    std::vector<void*> ln1, ln2, qkv, qk, att, hdact, hact;
    std::vector<float*> lse;
    void* lnf = nullptr;
    void* logits = nullptr;
    float* row_loss = nullptr;
    float* dres = nullptr;
    void* dres_lp = nullptr;
    void* dln = nullptr;
    void *dh = nullptr, *dO = nullptr, *dqkv = nullptr;
    // bf16 path: one copy per layer of dh and dqkv and one bf16 residual-
    // gradient copy per LayerNorm backward call, so that the main stream never
    // overwrites what a side-stream weight-gradient product still reads
    void *dres_lp_all = nullptr, *dh_all = nullptr, *dqkv_all = nullptr;
    float* attD = nullptr;
    // row-pass partial sums of every LayerNorm backward and bias column sum of
    // a backward pass, reduced together at its end (reduce_jobs)
    float *ln_part = nullptr, *cs_part = nullptr, *red_tmp = nullptr;
    size_t ln_part_stride = 0, cs_part_stride = 0;
    gk::RedJob* red_jobs = nullptr;
    int red_max_jobs = 0;
    double* gn_partial = nullptr;
    void* emb_scratch = nullptr;
    float* splitk = nullptr;
    size_t splitk_floats = 0;
    // split-K slices of the weight-gradient products that run on the side stream
    float* splitk_side = nullptr;
    size_t splitk_side_floats = 0;
    float *rope_cos = nullptr, *rope_sin = nullptr;
    // sampling: per-layer key and value caches [max_batch, block_size, d]
    // (act) and the one-token-per-sequence buffers of a decode step
    std::vector<void*> kcache, vcache;
    // FP8 head: e4m3 copies of the final LayerNorm output and of wte, their
    // scales [s_x, 1/s_x, s_w, 1/s_w] and the max-reduction partials
    uint8_t *xq = nullptr, *wq = nullptr;
    float *f8_scale = nullptr, *f8_part = nullptr;
    // Muon, for the n_layer matrices of one kind at a time: the directions u
    // (fp32, wide), the iterates X (two sets), A, A A and a I + b A + c A A
    // (act), per-tile sums of squares and the normalisations
    float* mu_u = nullptr;
    void *mu_x0 = nullptr, *mu_x1 = nullptr, *mu_a = nullptr, *mu_aa = nullptr, *mu_b = nullptr;
    float *mu_part = nullptr, *mu_scale = nullptr;
    int64_t mu_part_stride = 0;
    float *dec_x = nullptr, *dec_x2 = nullptr, *dec_mean = nullptr, *dec_rstd = nullptr, *dec_logits = nullptr;
    void *dec_y = nullptr, *dec_qkv = nullptr, *dec_qk = nullptr, *dec_att = nullptr, *dec_h1 = nullptr,
         *dec_h2 = nullptr;
    int32_t* err = nullptr;
    float *loss_last = nullptr, *loss_sum = nullptr, *gnorm = nullptr, *coef = nullptr;
    int32_t* nonfinite = nullptr;
    size_t bytes = 0;
};

struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base((char*)b) {}
    void* take(size_t bytes) {
        void* r = base ? base + off : nullptr;
        off += (bytes + 255) & ~size_t(255);
        return r;
    }
    template <typename T> T* arr(size_t n) { return (T*)take(sizeof(T) * n); }
};

bool qk_transform(const gpt_config& c) { return c.qk_rmsnorm || c.pos_encoding == GPT_POS_ROPE; }

Ws plan(const gpt_config& c, const Table& tb, void* base) {
    Ws w;
    Carver cv(base);
    const int64_t M = (int64_t)c.max_batch * c.block_size;
    const int64_t d = c.n_embd, F = c.mlp_hidden, Vp = c.padded_vocab_size, L = c.n_layer, H = c.n_head;
    const bool bf = c.precision == GPT_PREC_BF16;
    const size_t ab = bf ? 2 : 4;
    w.params = cv.arr<float>(tb.n_total);
    w.grads = cv.arr<float>(tb.n_total);
    w.m = cv.arr<float>(tb.n_total);
    w.v = cv.arr<float>(tb.n_total);
    if (bf) w.wbf = cv.take(2 * tb.n_decay);
    for (int l = 0; l < L; ++l) {
        w.x_in.push_back(cv.arr<float>(M * d));
        w.x_mid.push_back(cv.arr<float>(M * d));
        w.ln1.push_back(cv.take(ab * M * d));
        w.ln2.push_back(cv.take(ab * M * d));
        w.qkv.push_back(cv.take(ab * M * 3 * d));
        w.qk.push_back(qk_transform(c) ? cv.take(ab * M * 2 * d) : nullptr);
        w.att.push_back(cv.take(ab * M * d));
        w.lse.push_back(cv.arr<float>(M * H));
        w.hdact.push_back(cv.take(ab * M * F));
        w.hact.push_back(cv.take(ab * M * F));
    }
    w.x_fin = cv.arr<float>(M * d);
    w.ln_mean = cv.arr<float>((2 * L + 1) * M);
    w.ln_rstd = cv.arr<float>((2 * L + 1) * M);
    w.lnf = cv.take(ab * M * d);
    w.logits = cv.take(ab * M * Vp);
    w.row_loss = cv.arr<float>(M);
    w.dres = cv.arr<float>(M * d);
    if (bf) {
        w.dres_lp = cv.take(ab * M * d);
        w.dres_lp_all = cv.take(ab * M * d * (2 * L + 1));
        w.dh_all = cv.take(ab * M * F * L);
        w.dqkv_all = cv.take(ab * M * 3 * d * L);
    }
    w.dln = cv.take(ab * M * d);   // gradient at a LayerNorm output (bf16 on the bf16 path)
    w.dh = cv.take(ab * M * F);
    w.dO = cv.take(ab * M * d);
    w.dqkv = cv.take(ab * M * 3 * d);
    w.attD = cv.arr<float>(M * H);
    {
        const int64_t maxN = std::max<int64_t>(3 * d, F);
        const int nbl = gk::layernorm_bwd_num_partials((int)M), npc = gk::colsum_num_partials((int)M);
        // bias column sums come from colsum_rows (npc rows) or from the
        // attention backward (one row per 128-row block of each sequence)
        const int npa = c.max_batch * ((c.block_size + 127) / 128);
        w.ln_part_stride = (size_t)3 * nbl * d;
        w.cs_part_stride = (size_t)std::max(npc, npa) * maxN;
        w.ln_part = cv.arr<float>((size_t)(2 * L + 1) * w.ln_part_stride);
        w.cs_part = cv.arr<float>((size_t)(2 * L) * w.cs_part_stride);
        w.red_max_jobs = (int)((2 * L + 1) * 3 + 2 * L);
        w.red_tmp = cv.arr<float>(
            gk::reduce_jobs_tmp_floats(w.red_max_jobs, std::max({nbl, npc, npa}), (int)std::max(d, maxN)));
        w.red_jobs = (gk::RedJob*)cv.take(sizeof(gk::RedJob) * w.red_max_jobs);
    }
    w.gn_partial = cv.arr<double>(1024);
    w.emb_scratch = cv.take(gk::embed_bwd_scratch_bytes((int)M, (int)d));
    // fp32 slices of split-K products (matrix-core path only): weight
    // gradients, the N = d products over M rows, and the tied head's gradient
    w.splitk_floats = bf ? (size_t)std::max<int64_t>({8 * std::max<int64_t>(3 * d * d, F * d), 4 * M * d, 2 * Vp * d}) : 0;
    w.splitk = cv.arr<float>(w.splitk_floats);
    w.splitk_side_floats = bf ? (size_t)(8 * std::max<int64_t>(3 * d * d, F * d)) : 0;
    w.splitk_side = cv.arr<float>(w.splitk_side_floats);
    if (c.pos_encoding == GPT_POS_ROPE) {
        int64_t half = (d / H) / 2;
        w.rope_cos = cv.arr<float>(c.block_size * half);
        w.rope_sin = cv.arr<float>(c.block_size * half);
    }
    if (c.head_fp8) {
        w.xq = cv.arr<uint8_t>(M * d);
        w.wq = cv.arr<uint8_t>(Vp * d);
        w.f8_scale = cv.arr<float>(4);
        w.f8_part = cv.arr<float>(2048);
    }
    {
        // hidden matrices: [3d, d], [d, d], [F, d], [d, F]; the wide side m <= d
        const int64_t mn = L * std::max<int64_t>(3 * d * d, F * d), mm = L * d * d;
        const int64_t np = std::max({gk::muon_part_floats((int)(3 * d), (int)d), gk::muon_part_floats((int)F, (int)d),
                                     gk::muon_part_floats((int)d, (int)d)});
        w.mu_u = cv.arr<float>(mn);
        w.mu_x0 = cv.take(ab * mn);
        w.mu_x1 = cv.take(ab * mn);
        w.mu_a = cv.take(ab * mm);
        w.mu_aa = cv.take(ab * mm);
        w.mu_b = cv.take(ab * mm);
        w.mu_part = cv.arr<float>(L * np);
        w.mu_part_stride = np;
        w.mu_scale = cv.arr<float>(L);
    }
    for (int l = 0; l < L; ++l) {
        w.kcache.push_back(cv.take(ab * M * d));
        w.vcache.push_back(cv.take(ab * M * d));
    }
    {
        const int64_t Bm = c.max_batch;
        w.dec_x = cv.arr<float>(Bm * d);
        w.dec_x2 = cv.arr<float>(Bm * d);
        w.dec_mean = cv.arr<float>(Bm);
        w.dec_rstd = cv.arr<float>(Bm);
        w.dec_logits = cv.arr<float>(Bm * Vp);
        w.dec_y = cv.take(ab * Bm * d);
        w.dec_qkv = cv.take(ab * Bm * 3 * d);
        w.dec_qk = cv.take(ab * Bm * 2 * d);
        w.dec_att = cv.take(ab * Bm * d);
        w.dec_h1 = cv.take(ab * Bm * F);
        w.dec_h2 = cv.take(ab * Bm * F);
    }
    w.err = cv.arr<int32_t>(4);
    w.loss_last = cv.arr<float>(4);
    w.loss_sum = cv.arr<float>(4);
    w.gnorm = cv.arr<float>(4);
    w.coef = cv.arr<float>(4);
    w.nonfinite = cv.arr<int32_t>(4);
    w.bytes = cv.off;
    return w;
}

gpt_status validate(const gpt_config* c, std::string* why) { return gpth::validate_config(c, why); }

// ---------------------------------------------------------------- timing

enum KClass {
    KC_EMBED_FWD, KC_LN_FWD, KC_GEMM_FWD, KC_GEMM_LMHEAD, KC_ATTN_FWD, KC_CE, KC_GEMM_DGRAD, KC_GEMM_WGRAD,
    KC_GEMM_LMHEAD_BWD, KC_LN_BWD, KC_COLSUM, KC_ATTN_BWD, KC_QK_PREP, KC_EMBED_BWD, KC_GRAD_NORM, KC_ADAMW,
    KC_MISC, KC_PARTIAL_REDUCE, KC_FP8_QUANT, KC_MUON, KC_COUNT
};
const char* kc_names[KC_COUNT] = {
    "embed_fwd", "layernorm_fwd", "gemm_fwd", "gemm_lm_head", "attention_fwd", "cross_entropy", "gemm_dgrad",
    "gemm_wgrad", "gemm_lm_head_bwd", "layernorm_bwd", "colsum", "attention_bwd", "qk_prep", "embed_bwd",
    "grad_norm", "adamw", "misc", "partial_reduce", "fp8_quantize", "muon"};

struct Pending { int cls; int name; hipEvent_t a, b; double flops, bytes; };
struct ClassStat { double ms = 0, flops = 0, bytes = 0; int64_t launches = 0; };
struct NameStat { std::string name; ClassStat st; };

}  // namespace

struct gpt_handle {
    gpt_config cfg;
    Table tb;
    Ws ws;
    hipStream_t stream = nullptr;
    bool grads_dirty = true;     // true: the next micro-step starts from zero
    int micro_count = 0;
    std::string last_error;
    uint32_t timing_mask = 0;
    std::vector<Pending> pending;
    std::vector<hipEvent_t> free_events;
    ClassStat stats[KC_COUNT];
    std::vector<NameStat> names;     // per kernel (instantiation) name
    std::string filter;              // also time launches of this kernel name
    std::vector<gk::RedJob> jobs;    // this backward pass's deferred reductions
    std::vector<gk::RedJob> jobs_dev;   // the table last copied to the workspace
    // side stream (default priority) for the embedding backward's token sort,
    // which depends on the tokens only and overlaps the forward pass
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    // dependencies between the backward pass's main stream and the weight-
    // gradient products it runs on the side stream
    hipEvent_t ev_dep[8] = {};
};

namespace {

gpt_status fail(gpt_handle* h, gpt_status s, const std::string& msg) {
    if (h) h->last_error = msg;
    return s;
}

gpt_status hip_check(gpt_handle* h, hipError_t e, const char* what) {
    if (e == hipSuccess) return GPT_OK;
    return fail(h, GPT_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

hipEvent_t get_event(gpt_handle* h) {
    if (!h->free_events.empty()) { hipEvent_t e = h->free_events.back(); h->free_events.pop_back(); return e; }
    hipEvent_t e;
    (void)hipEventCreate(&e);
    return e;
}

int name_index(gpt_handle* h, const char* name) {
    for (size_t i = 0; i < h->names.size(); ++i)
        if (h->names[i].name == name) return (int)i;
    h->names.push_back({name, ClassStat()});
    return (int)h->names.size() - 1;
}

// Brackets one kernel launch with events when its class is enabled or its
// kernel name is the filter; the statistics count timed launches only.
struct Timed {
    gpt_handle* h;
    int cls;
    const char* name;
    double flops, bytes;
    hipStream_t s;     // the stream the bracketed launch goes to
    hipEvent_t a = nullptr;
    Timed(gpt_handle* h_, int cls_, double flops_, double bytes_, const char* name_ = nullptr,
          hipStream_t s_ = nullptr)
        : h(h_), cls(cls_), name(name_ ? name_ : kc_names[cls_]), flops(flops_), bytes(bytes_),
          s(s_ ? s_ : h_->stream) {
        if ((h->timing_mask & (1u << cls)) || (!h->filter.empty() && h->filter == name)) {
            a = get_event(h);
            (void)hipEventRecord(a, s);
        }
    }
    ~Timed() {
        if (a) {
            hipEvent_t b = get_event(h);
            (void)hipEventRecord(b, s);
            h->pending.push_back({cls, name_index(h, name), a, b, flops, bytes});
        }
    }
};

void drain_timing(gpt_handle* h) {
    if (h->pending.empty()) return;
    (void)hipStreamSynchronize(h->stream);
    if (h->side) (void)hipStreamSynchronize(h->side);
    for (auto& p : h->pending) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            for (ClassStat* c : {&h->stats[p.cls], &h->names[p.name].st}) {
                c->ms += ms;
                c->flops += p.flops;
                c->bytes += p.bytes;
                c->launches += 1;
            }
        }
        h->free_events.push_back(p.a);
        h->free_events.push_back(p.b);
    }
    h->pending.clear();
}

float* P(gpt_handle* h, int idx) { return h->ws.params + h->tb.t[idx].offset; }
float* G(gpt_handle* h, int idx) { return h->ws.grads + h->tb.t[idx].offset; }
// weight operand of the matrix products: bf16 copy or fp32 master
const void* Wop(gpt_handle* h, int idx) {
    if (h->cfg.precision == GPT_PREC_BF16) return (const char*)h->ws.wbf + 2 * h->tb.t[idx].offset;
    return P(h, idx);
}

// On the handle's stream with the main split-K scratch, or (side = true) on the
// side stream with its own scratch; timing events go to the launch's stream.
void run_gemm(gpt_handle* h, int cls, const gk::Gemm& g, bool side = false) {
    const double ab = g.in_bf ? 2 : 4, cb = g.c_bf ? 2 : 4;
    const double bytes = ab * ((double)g.M * g.K + (double)g.K * g.N) + cb * (double)g.M * g.N;
    float* scratch = side ? h->ws.splitk_side : h->ws.splitk;
    const size_t nscratch = side ? h->ws.splitk_side_floats : h->ws.splitk_floats;
    hipStream_t s = side ? h->side : h->stream;
    const gk::GemmPlan plan = gk::gemm_plan(g, nscratch);
    {
        Timed t(h, cls, 2.0 * g.M * g.N * g.K, bytes, plan.name, s);
        gk::gemm_main(g, plan, scratch, s);
    }
    if (plan.splits > 1) {
        Timed t(h, cls, 0, 4.0 * plan.splits * g.M * g.N + cb * (double)g.M * g.N, "splitk_reduce_kernel", s);
        gk::gemm_finish(g, plan, scratch, s);
    }
}

// the products of a sampling step: the skinny kernel where it applies
void run_decode_gemm(gpt_handle* h, const gk::Gemm& g) {
    if (gk::skinny_gemm_ok(g)) {
        Timed t(h, KC_MISC, 2.0 * g.M * g.N * g.K, 2.0 * ((double)g.M * g.K + (double)g.N * g.K), "skinny_gemm_kernel");
        gk::skinny_gemm(g, h->stream);
    } else {
        run_gemm(h, KC_MISC, g);
    }
}

gk::Gemm mk_gemm(gpt_handle* h, int M, int N, int K, const void* A, int64_t lda, bool a_kc, const void* B,
                 int64_t ldb, bool b_kc, void* C, int64_t ldc, bool c_bf, int epi) {
    gk::Gemm g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.a_kc = a_kc;
    g.B = B; g.ldb = ldb; g.b_kc = b_kc;
    g.C = C; g.ldc = ldc; g.c_bf = c_bf;
    g.epi = epi;
    g.act = h->cfg.mlp_act == GPT_ACT_RELU2 ? 1 : 0;
    g.in_bf = h->cfg.precision == GPT_PREC_BF16;
    return g;
}

int window_of(const gpt_config& c, int l) { return (l % 2 == 0) ? c.window_even : c.window_odd; }

double attn_pairs(int B, int T, int H, int W) {
    double p = 0;
    if (W <= 0 || W >= T) p = (double)T * (T + 1) / 2;
    else p = (double)W * (W + 1) / 2 + (double)(T - W) * W;
    return p * B * H;
}

gpt_status sync_and_check(gpt_handle* h) {
    gpt_status s = hip_check(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
    if (s != GPT_OK) return s;
    int32_t err = 0;
    s = hip_check(h, hipMemcpy(&err, h->ws.err, sizeof(int32_t), hipMemcpyDeviceToHost), "read error flag");
    if (s != GPT_OK) return s;
    if (err) {
        int32_t zero = 0;
        (void)hipMemcpy(h->ws.err, &zero, sizeof(int32_t), hipMemcpyHostToDevice);
        return fail(h, GPT_ERR_TOKEN_RANGE, "a token or target id is outside [0, padded_vocab_size)");
    }
    return GPT_OK;
}

// Forward pass of one micro-batch [B, T] up to the final LayerNorm (w.lnf),
// keeping every activation the backward pass and the key/value caches read.
void forward_pass(gpt_handle* h, const int32_t* tok, int B, int T) {
    const gpt_config& c = h->cfg;
    Ws& w = h->ws;
    const Table& tb = h->tb;
    hipStream_t st = h->stream;
    const int M = B * T, d = c.n_embd, F = c.mlp_hidden, Vp = c.padded_vocab_size, H = c.n_head;
    const int hd = d / H, L = c.n_layer;
    const bool bf = c.precision == GPT_PREC_BF16;
    const double ab = bf ? 2 : 4;
    const bool qkt = qk_transform(c);
    {
        Timed t(h, KC_EMBED_FWD, 0, (double)M * d * (tb.wpe >= 0 ? 12 : 8) + 4.0 * M);
        gk::embed_fwd(tok, P(h, tb.wte), tb.wpe >= 0 ? P(h, tb.wpe) : nullptr, w.x_in[0], M, T, d, Vp, w.err, st);
    }
    for (int l = 0; l < L; ++l) {
        const LayerIdx& li = tb.layers[l];
        float* mean1 = w.ln_mean + (size_t)(2 * l) * M;
        float* rstd1 = w.ln_rstd + (size_t)(2 * l) * M;
        float* mean2 = w.ln_mean + (size_t)(2 * l + 1) * M;
        float* rstd2 = w.ln_rstd + (size_t)(2 * l + 1) * M;
        {
            Timed t(h, KC_LN_FWD, 0, (double)M * d * (4 + ab) + 8.0 * M);
            gk::layernorm_fwd(bf, w.x_in[l], P(h, li.ln1_w), P(h, li.ln1_b), w.ln1[l], mean1, rstd1, M, d, c.ln_eps, st);
        }
        {
            gk::Gemm g = mk_gemm(h, M, 3 * d, d, w.ln1[l], d, true, Wop(h, li.attn_w), d, true, w.qkv[l], 3 * d, bf,
                                 gk::EPI_BIAS);
            g.bias = P(h, li.attn_b);
            run_gemm(h, KC_GEMM_FWD, g);
        }
        const void *q = w.qkv[l], *k = (const char*)w.qkv[l] + (size_t)ab * d;
        int64_t ldq = 3 * d, ldk = 3 * d;
        if (qkt) {
            Timed t(h, KC_QK_PREP, 0, (double)M * 2 * d * 2 * ab);
            gk::qk_prep_fwd(bf, w.qkv[l], w.qk[l], w.rope_cos, w.rope_sin, M, T, H, hd, c.qk_rmsnorm,
                            c.pos_encoding == GPT_POS_ROPE, c.qk_norm_eps, st);
            q = w.qk[l];
            k = (const char*)w.qk[l] + (size_t)ab * d;
            ldq = ldk = 2 * d;
        }
        gk::Attn a{};
        a.B = B; a.T = T; a.H = H; a.hd = hd; a.window = window_of(c, l);
        a.q = q; a.k = k; a.v = (const char*)w.qkv[l] + (size_t)ab * 2 * d;
        a.ldq = ldq; a.ldk = ldk; a.ldv = 3 * d;
        a.o = w.att[l]; a.ldo = d; a.lse = w.lse[l]; a.bf = bf;
        {
            double pairs = attn_pairs(B, T, H, a.window);
            Timed t(h, KC_ATTN_FWD, 4.0 * hd * pairs, (double)M * d * 4 * ab + 4.0 * M * H);
            gk::attention_fwd(a, st);
        }
        {
            gk::Gemm g = mk_gemm(h, M, d, d, w.att[l], d, true, Wop(h, li.proj_w), d, true, w.x_mid[l], d, false,
                                 gk::EPI_BIAS_RESID);
            g.bias = P(h, li.proj_b);
            g.resid = w.x_in[l];
            run_gemm(h, KC_GEMM_FWD, g);
        }
        {
            Timed t(h, KC_LN_FWD, 0, (double)M * d * (4 + ab) + 8.0 * M);
            gk::layernorm_fwd(bf, w.x_mid[l], P(h, li.ln2_w), P(h, li.ln2_b), w.ln2[l], mean2, rstd2, M, d, c.ln_eps, st);
        }
        {
            gk::Gemm g = mk_gemm(h, M, F, d, w.ln2[l], d, true, Wop(h, li.fc_w), d, true, w.hdact[l], F, bf,
                                 gk::EPI_BIAS_ACT);
            g.bias = P(h, li.fc_b);
            g.C2 = w.hact[l];
            run_gemm(h, KC_GEMM_FWD, g);
        }
        {
            float* xo = (l + 1 < L) ? w.x_in[l + 1] : w.x_fin;
            gk::Gemm g = mk_gemm(h, M, d, F, w.hact[l], F, true, Wop(h, li.mp_w), F, true, xo, d, false,
                                 gk::EPI_BIAS_RESID);
            g.bias = P(h, li.mp_b);
            g.resid = w.x_mid[l];
            run_gemm(h, KC_GEMM_FWD, g);
        }
    }
    float* meanf = w.ln_mean + (size_t)(2 * L) * M;
    float* rstdf = w.ln_rstd + (size_t)(2 * L) * M;
    {
        Timed t(h, KC_LN_FWD, 0, (double)M * d * (4 + ab) + 8.0 * M);
        gk::layernorm_fwd(bf, w.x_fin, P(h, tb.lnf_w), P(h, tb.lnf_b), w.lnf, meanf, rstdf, M, d, c.ln_eps, st);
    }
}

gpt_status copy_tensor(gpt_handle* h, float* dst, const float* src, int64_t count, int dir_dev_to_host_buf,
                       int on_device) {
    (void)dir_dev_to_host_buf;
    hipMemcpyKind kind = on_device ? hipMemcpyDeviceToDevice : hipMemcpyDefault;
    gpt_status s = hip_check(h, hipMemcpyAsync(dst, src, sizeof(float) * count, kind, h->stream), "hipMemcpyAsync");
    if (s != GPT_OK) return s;
    return hip_check(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
}

gpt_status check_idx(const gpt_handle* h, int32_t idx, int64_t count) {
    if (!h || idx < 0 || idx >= (int32_t)h->tb.t.size()) return GPT_ERR_INVALID_ARGUMENT;
    if (count != h->tb.t[idx].numel) return GPT_ERR_INVALID_ARGUMENT;
    return GPT_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================

extern "C" {

gpt_status gpt_config_default(gpt_config* c) {
    if (!c) return GPT_ERR_INVALID_ARGUMENT;
    gpth::config_defaults(c);
    return GPT_OK;
}

gpt_status gpt_workspace_bytes(const gpt_config* cfg, size_t* bytes) {
    if (!bytes) return GPT_ERR_INVALID_ARGUMENT;
    gpt_status s = validate(cfg, nullptr);
    if (s != GPT_OK) return s;
    Table tb = build_table(*cfg);
    *bytes = plan(*cfg, tb, nullptr).bytes;
    return GPT_OK;
}

gpt_status gpt_create(const gpt_config* cfg, uint64_t seed, void* d_ws, size_t ws_bytes, void* stream,
                      gpt_handle** out) {
    if (!out || !d_ws) return GPT_ERR_INVALID_ARGUMENT;
    *out = nullptr;
    std::string why;
    gpt_status s = validate(cfg, &why);
    if (s != GPT_OK) return s;
    if ((uintptr_t)d_ws % 256) return GPT_ERR_INVALID_ARGUMENT;
    Table tb = build_table(*cfg);
    Ws probe = plan(*cfg, tb, nullptr);
    if (ws_bytes < probe.bytes) return GPT_ERR_WORKSPACE_TOO_SMALL;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GPT_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GPT_ERR_DEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return GPT_ERR_UNSUPPORTED;

    gpt_handle* h = new gpt_handle();
    h->cfg = *cfg;
    h->tb = tb;
    h->ws = plan(*cfg, tb, d_ws);
    h->stream = (hipStream_t)stream;
    Ws& w = h->ws;
    hipStream_t st = h->stream;
    const int64_t n = tb.n_total;
    gk::fill_f32(w.params, n, 0.f, st);
    gk::fill_f32(w.grads, n, 0.f, st);
    gk::fill_f32(w.m, n, 0.f, st);
    gk::fill_f32(w.v, n, 0.f, st);
    const double L = cfg->n_layer;
    for (size_t i = 0; i < tb.t.size(); ++i) {
        const TensorInfo& ti = tb.t[i];
        float* dst = w.params + ti.offset;
        if (ti.init == INIT_ONE) gk::fill_f32(dst, ti.numel, 1.f, st);
        else if (ti.init == INIT_ZERO || (ti.init == INIT_PROJ && cfg->zero_init_proj)) continue;
        else {
            double std = cfg->init_std * (ti.init == INIT_PROJ ? std::pow(2.0 * L, -0.5) : 1.0);
            gk::init_normal(dst, ti.numel, seed, (uint64_t)i, std, st);
        }
    }
    if (w.wbf) gk::f32_to_bf16(w.wbf, w.params, tb.n_decay, st);
    if (w.rope_cos)
        gk::rope_tables(w.rope_cos, w.rope_sin, cfg->block_size, cfg->n_embd / cfg->n_head, cfg->rope_base, st);
    gk::fill_i32(w.err, 4, 0, st);
    gk::fill_f32(w.loss_sum, 4, 0.f, st);
    gk::fill_f32(w.loss_last, 4, 0.f, st);
    gk::fill_i32(w.nonfinite, 4, 0, st);
    s = hip_check(h, hipGetLastError(), "kernel launch");
    if (s == GPT_OK) s = hip_check(h, hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking), "hipStreamCreate");
    if (s == GPT_OK) s = hip_check(h, hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming), "hipEventCreate");
    if (s == GPT_OK) s = hip_check(h, hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming), "hipEventCreate");
    for (hipEvent_t& e : h->ev_dep)
        if (s == GPT_OK) s = hip_check(h, hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreate");
    if (s != GPT_OK) {
        (void)hipStreamSynchronize(st);
        if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
        if (h->ev_join) (void)hipEventDestroy(h->ev_join);
        for (hipEvent_t e : h->ev_dep)
            if (e) (void)hipEventDestroy(e);
        if (h->side) (void)hipStreamDestroy(h->side);
        delete h;
        return s;
    }
    h->grads_dirty = true;
    *out = h;
    return GPT_OK;
}

gpt_status gpt_destroy(gpt_handle* h) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    if (!h->pending.empty()) (void)hipStreamSynchronize(h->stream);
    if (h->side) (void)hipStreamSynchronize(h->side);
    for (auto& p : h->pending) { (void)hipEventDestroy(p.a); (void)hipEventDestroy(p.b); }
    for (auto e : h->free_events) (void)hipEventDestroy(e);
    if (h->side) (void)hipStreamSynchronize(h->side);
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    if (h->ev_join) (void)hipEventDestroy(h->ev_join);
    for (hipEvent_t e : h->ev_dep)
        if (e) (void)hipEventDestroy(e);
    if (h->side) (void)hipStreamDestroy(h->side);
    delete h;
    return GPT_OK;
}

gpt_status gpt_set_stream(gpt_handle* h, void* stream) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    // pending timing events were recorded on the old stream: collect them
    // before switching (not on every call with the same stream, which would
    // make the host wait for the GPU between a step's calls)
    if ((hipStream_t)stream != h->stream) drain_timing(h);
    h->stream = (hipStream_t)stream;
    return GPT_OK;
}

gpt_status gpt_forward_backward(gpt_handle* h, const int32_t* tok, const int32_t* tgt, int32_t B, int32_t T,
                                float grad_scale, float* h_loss) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    const gpt_config& c = h->cfg;
    if (!tok || !tgt) return fail(h, GPT_ERR_INVALID_ARGUMENT, "null token or target buffer");
    if (B < 1 || B > c.max_batch) return fail(h, GPT_ERR_INVALID_ARGUMENT, "B must be in [1, max_batch]");
    if (T < 1 || T > c.block_size)
        return fail(h, GPT_ERR_INVALID_ARGUMENT, "T must be in [1, block_size]: cannot forward a longer sequence");
    if (!std::isfinite(grad_scale)) return fail(h, GPT_ERR_INVALID_ARGUMENT, "grad_scale not finite");
    Ws& w = h->ws;
    const Table& tb = h->tb;
    hipStream_t st = h->stream;
    const int M = B * T, d = c.n_embd, F = c.mlp_hidden, Vp = c.padded_vocab_size, H = c.n_head;
    const int hd = d / H, L = c.n_layer;
    const bool bf = c.precision == GPT_PREC_BF16;
    const double ab = bf ? 2 : 4;
    const bool qkt = qk_transform(c);
    const int gelu_or_relu = c.mlp_act == GPT_ACT_RELU2 ? 1 : 0;
    (void)gelu_or_relu;

    // The first micro-step after an update (gradients logically zero) writes
    // every gradient instead of adding to it: the weight-gradient products
    // store, the tied head's product stores all of wte before the embedding
    // rows are added to it, and the bias / LayerNorm reductions, dwpe and the
    // loss sum overwrite. Every element of a tensor is written exactly once by
    // one of them, so no zero fill is needed (0 + x and x are the same value;
    // the padding between tensors is zero from creation and never written).
    const bool first = h->grads_dirty;
    if (h->grads_dirty) {
        h->grads_dirty = false;
        h->micro_count = 0;
    }
    const int wg_epi = first ? gk::EPI_STORE : gk::EPI_ACCUM;
    // token sort of the embedding backward, on the side stream: it waits for
    // the work queued so far on the main stream (the tokens), and the main
    // stream waits for it before the embedding gradient
    {
        gpt_status s = hip_check(h, hipEventRecord(h->ev_fork, st), "hipEventRecord");
        if (s == GPT_OK) s = hip_check(h, hipStreamWaitEvent(h->side, h->ev_fork, 0), "hipStreamWaitEvent");
        if (s != GPT_OK) return s;
        gk::embed_bwd_sort(tok, B, T, d, Vp, w.emb_scratch, h->side);
        s = hip_check(h, hipEventRecord(h->ev_join, h->side), "hipEventRecord");
        if (s != GPT_OK) return s;
    }
    // ------------------------------------------------------------ forward
    forward_pass(h, tok, B, T);
    float* meanf = w.ln_mean + (size_t)(2 * L) * M;
    float* rstdf = w.ln_rstd + (size_t)(2 * L) * M;
    if (c.head_fp8) {
        // e4m3 copies of both operands: scales at [2] (x) and [3] (wte), their
        // inverses at [0] and [1], which the product's store multiplies by
        {
            Timed t(h, KC_FP8_QUANT, 0, 3.0 * ((double)M + Vp) * d + 8.0 * 1024);
            gk::quantize_e4m3(w.lnf, (int64_t)M * d, w.xq, w.f8_scale + 2, w.f8_scale, w.f8_part, st);
            gk::quantize_e4m3(Wop(h, tb.wte), (int64_t)Vp * d, w.wq, w.f8_scale + 3, w.f8_scale + 1,
                              w.f8_part + 1024, st);
        }
        Timed t(h, KC_GEMM_LMHEAD, 2.0 * M * Vp * d, (double)M * d + (double)Vp * d + 2.0 * M * Vp,
                "gemm_mfma_kernel<256, 256, 64, 2, 1, 3, 2, 4, true, true, 0, 1, 0, false>");
        gk::gemm_f8(M, Vp, d, w.xq, d, w.wq, d, w.logits, Vp, w.f8_scale, st);
    } else {
        gk::Gemm g = mk_gemm(h, M, Vp, d, w.lnf, d, true, Wop(h, tb.wte), d, true, w.logits, Vp, bf, gk::EPI_STORE);
        run_gemm(h, KC_GEMM_LMHEAD, g);
    }
    {
        Timed t(h, KC_CE, 0, (double)M * Vp * 2 * ab + 8.0 * M);
        gk::cross_entropy(bf, w.logits, tgt, w.row_loss, M, Vp, grad_scale / (float)M, c.logit_softcap, w.err, st);
        gk::mean_loss(w.row_loss, M, w.loss_last, w.loss_sum, st, first);
    }
    // ------------------------------------------------------------ backward
    // The weight-gradient products (they only read activations and upstream
    // gradients) run on the side stream, overlapping the input-gradient chain.
    // They read per-layer copies of dh, dqkv and the bf16 residual gradient,
    // so the main stream never waits for them inside the pass, and they wait
    // for two events per layer (after the MLP input gradient and after the
    // attention backward): every event operation on the main stream costs
    // about 12 us of idle GPU between its kernels. Not while per-class timing
    // is on (its class totals assume one stream).
    const bool conc = bf && h->timing_mask == 0;
    enum { E_DH = 0, E_DQKV, E_DZ, S_END, E_MAIN_END };
    auto record = [&](int e, hipStream_t s_) { if (conc) (void)hipEventRecord(h->ev_dep[e], s_); };
    auto wait_ev = [&](hipStream_t s_, int e) { if (conc) (void)hipStreamWaitEvent(s_, h->ev_dep[e], 0); };
    hipStream_t sw = conc ? h->side : st;
    {
        // the tied head's weight gradient (dz^T lnf) goes to the side stream
        // first, beside its input gradient and the layers' input-gradient chain
        record(E_DZ, st);
        wait_ev(sw, E_DZ);
        gk::Gemm g2 = mk_gemm(h, Vp, d, M, w.logits, Vp, false, w.lnf, d, false, G(h, tb.wte), d, false, wg_epi);
        run_gemm(h, KC_GEMM_LMHEAD_BWD, g2, conc);
        gk::Gemm g = mk_gemm(h, M, d, Vp, w.logits, Vp, true, Wop(h, tb.wte), d, false, w.dln, d, bf, gk::EPI_STORE);
        run_gemm(h, KC_GEMM_LMHEAD_BWD, g);
    }
    // residual gradient as a matrix-product operand: its bf16 copy (per
    // LayerNorm backward call while the side stream runs) or the fp32 buffer
    void* dR = bf ? w.dres_lp : (void*)w.dres;
    // LayerNorm backward row passes and bias column sums leave their partial
    // sums in per-call slots; one reduce_jobs at the end of the pass sums them
    h->jobs.clear();
    const int nbl = gk::layernorm_bwd_num_partials(M), npc = gk::colsum_num_partials(M);
    const int npa = B * ((T + 127) / 128);   // row blocks of the attention backward's column sums
    int n_ln = 0, n_cs = 0;
    auto ln_bwd = [&](const float* x, const float* mean, const float* rstd, const float* g, bool overwrite, float* dg,
                      float* db, float* dcol) {
        Timed t(h, KC_LN_BWD, 0, (double)M * d * ((overwrite ? 8 : 12) + 2 * ab) + 8.0 * M + 12.0 * nbl * d);
        float* part = w.ln_part + (size_t)(n_ln++) * w.ln_part_stride;
        if (conc) dR = (char*)w.dres_lp_all + (size_t)(n_ln - 1) * (size_t)ab * M * d;
        gk::layernorm_bwd_rows(bf, w.dln, bf, x, mean, rstd, g, w.dres, bf ? dR : nullptr, overwrite, part, M, d, st);
        float* outs[3] = {dg, db, dcol};
        for (int q = 0; q < 3; ++q)
            if (outs[q]) h->jobs.push_back({part + (size_t)q * nbl * d, outs[q], nbl, d});
    };
    auto col_sum = [&](const void* Y, int N, float* out) {
        Timed t(h, KC_COLSUM, 0, (double)ab * M * N + 4.0 * npc * N);
        float* part = w.cs_part + (size_t)(n_cs++) * w.cs_part_stride;
        gk::colsum_rows(bf, Y, N, M, N, part, st);
        h->jobs.push_back({part, out, npc, N});
    };
    ln_bwd(w.x_fin, meanf, rstdf, P(h, tb.lnf_w), true, G(h, tb.lnf_w), G(h, tb.lnf_b), G(h, tb.layers[L - 1].mp_b));
    for (int l = L - 1; l >= 0; --l) {
        const LayerIdx& li = tb.layers[l];
        float* mean1 = w.ln_mean + (size_t)(2 * l) * M;
        float* rstd1 = w.ln_rstd + (size_t)(2 * l) * M;
        float* mean2 = w.ln_mean + (size_t)(2 * l + 1) * M;
        float* rstd2 = w.ln_rstd + (size_t)(2 * l + 1) * M;
        // MLP branch
        bool fc_b_fused = false;   // fc bias gradient from the dgrad epilogue's column sums
        void* dh = conc ? (char*)w.dh_all + (size_t)l * (size_t)ab * M * F : w.dh;
        void* dqkv = conc ? (char*)w.dqkv_all + (size_t)l * (size_t)ab * M * 3 * d : w.dqkv;
        void* dR_mlp = dR;   // the mp products' operand (this layer's output gradient)
        {
            gk::Gemm g = mk_gemm(h, M, F, d, dR, d, true, Wop(h, li.mp_w), F, false, dh, F, bf, gk::EPI_ACT_GRAD);
            g.aux = w.hdact[l];
            const gk::GemmPlan pl = gk::gemm_plan(g, w.splitk_floats);
            if (pl.bm > 0) {
                g.cpart = w.cs_part + (size_t)(n_cs++) * w.cs_part_stride;
                h->jobs.push_back({g.cpart, G(h, li.fc_b), (M + pl.bm - 1) / pl.bm, F});
                fc_b_fused = true;
            }
            run_gemm(h, KC_GEMM_DGRAD, g);
            record(E_DH, st);
            wait_ev(sw, E_DH);
            gk::Gemm g2 = mk_gemm(h, d, F, M, dR_mlp, d, false, w.hact[l], F, false, G(h, li.mp_w), F, false, wg_epi);
            run_gemm(h, KC_GEMM_WGRAD, g2, conc);
        }
        {
            gk::Gemm g = mk_gemm(h, M, d, F, dh, F, true, Wop(h, li.fc_w), d, false, w.dln, d, bf, gk::EPI_STORE);
            run_gemm(h, KC_GEMM_DGRAD, g);
            gk::Gemm g2 = mk_gemm(h, F, d, M, dh, F, false, w.ln2[l], d, false, G(h, li.fc_w), d, false, wg_epi);
            run_gemm(h, KC_GEMM_WGRAD, g2, conc);
        }
        if (!fc_b_fused) col_sum(dh, F, G(h, li.fc_b));
        ln_bwd(w.x_mid[l], mean2, rstd2, P(h, li.ln2_w), false, G(h, li.ln2_w), G(h, li.ln2_b), G(h, li.proj_b));
        void* dR_attn = dR;   // the proj products' operand
        // attention branch
        {
            gk::Gemm g = mk_gemm(h, M, d, d, dR_attn, d, true, Wop(h, li.proj_w), d, false, w.dO, d, bf, gk::EPI_STORE);
            run_gemm(h, KC_GEMM_DGRAD, g);
        }
        const void *q = w.qkv[l], *k = (const char*)w.qkv[l] + (size_t)ab * d;
        int64_t ldq = 3 * d, ldk = 3 * d;
        if (qkt) {
            q = w.qk[l];
            k = (const char*)w.qk[l] + (size_t)ab * d;
            ldq = ldk = 2 * d;
        }
        gk::Attn a{};
        a.B = B; a.T = T; a.H = H; a.hd = hd; a.window = window_of(c, l);
        a.q = q; a.k = k; a.v = (const char*)w.qkv[l] + (size_t)ab * 2 * d;
        a.ldq = ldq; a.ldk = ldk; a.ldv = 3 * d;
        a.o = w.att[l]; a.ldo = d; a.lse = w.lse[l]; a.bf = bf;
        a.dO = w.dO; a.lddo = d; a.D = w.attD; a.Dout = w.attD;
        a.dq = dqkv; a.dk = (char*)dqkv + (size_t)ab * d; a.dv = (char*)dqkv + (size_t)ab * 2 * d; a.ldd = 3 * d;
        // qkv bias gradient: column sums of dqkv, from the attention backward itself
        // unless the q/k transform still changes dq and dk afterwards
        float* qkv_part = w.cs_part + (size_t)(n_cs++) * w.cs_part_stride;
        bool attn_b_fused = false;
        if (!qkt) a.cpart = qkv_part;
        {
            double pairs = attn_pairs(B, T, H, a.window);
            Timed t(h, KC_ATTN_BWD, 8.0 * hd * pairs, (double)M * d * 8 * ab + 8.0 * M * H);
            attn_b_fused = gk::attention_bwd(a, st) && a.cpart;
        }
        if (attn_b_fused) h->jobs.push_back({qkv_part, G(h, li.attn_b), npa, 3 * d});
        if (qkt) {
            Timed t(h, KC_QK_PREP, 0, (double)M * 2 * d * 3 * ab);
            gk::qk_prep_bwd(bf, w.qkv[l], dqkv, w.rope_cos, w.rope_sin, M, T, H, hd, c.qk_rmsnorm,
                            c.pos_encoding == GPT_POS_ROPE, c.qk_norm_eps, st);
        }
        record(E_DQKV, st);
        {
            gk::Gemm g = mk_gemm(h, M, d, 3 * d, dqkv, 3 * d, true, Wop(h, li.attn_w), d, false, w.dln, d, bf,
                                 gk::EPI_STORE);
            run_gemm(h, KC_GEMM_DGRAD, g);
            wait_ev(sw, E_DQKV);
            gk::Gemm g2 = mk_gemm(h, d, d, M, dR_attn, d, false, w.att[l], d, false, G(h, li.proj_w), d, false,
                                  wg_epi);
            run_gemm(h, KC_GEMM_WGRAD, g2, conc);
            gk::Gemm g3 = mk_gemm(h, 3 * d, d, M, dqkv, 3 * d, false, w.ln1[l], d, false, G(h, li.attn_w), d, false,
                                  wg_epi);
            run_gemm(h, KC_GEMM_WGRAD, g3, conc);
        }
        if (!attn_b_fused) {
            Timed t(h, KC_COLSUM, 0, (double)ab * M * 3 * d + 4.0 * npc * 3 * d);
            gk::colsum_rows(bf, dqkv, 3 * d, M, 3 * d, qkv_part, st);
            h->jobs.push_back({qkv_part, G(h, li.attn_b), npc, 3 * d});
        }
        ln_bwd(w.x_in[l], mean1, rstd1, P(h, li.ln1_w), false, G(h, li.ln1_w), G(h, li.ln1_b),
               l > 0 ? G(h, tb.layers[l - 1].mp_b) : nullptr);
    }
    // The bias / LayerNorm reductions read partial sums written on the main
    // stream only, so they run there at once; the embedding gradient (after the
    // tied head's product and the token sort, both earlier on the side stream,
    // and the main stream's last LayerNorm backward, which wrote dres) runs on
    // the side stream beside them; then the main stream waits for the side.
    record(E_MAIN_END, st);
    if (!h->jobs.empty()) {
        auto same = [](const gk::RedJob& a, const gk::RedJob& b) {
            return a.part == b.part && a.out == b.out && a.np == b.np && a.n == b.n;
        };
        const bool changed = h->jobs.size() != h->jobs_dev.size() ||
                             !std::equal(h->jobs.begin(), h->jobs.end(), h->jobs_dev.begin(), same);
        if (changed) {
            if ((int)h->jobs.size() > w.red_max_jobs) return fail(h, GPT_ERR_UNSUPPORTED, "reduction table overflow");
            // the previous pass's reduction may still read the table
            gpt_status s = hip_check(h, hipStreamSynchronize(st), "hipStreamSynchronize");
            if (s != GPT_OK) return s;
            s = hip_check(h, hipMemcpy(w.red_jobs, h->jobs.data(), sizeof(gk::RedJob) * h->jobs.size(),
                                       hipMemcpyHostToDevice), "copy reduction table");
            if (s != GPT_OK) return s;
            h->jobs_dev = h->jobs;
        }
        double bytes = 0;
        for (const gk::RedJob& j : h->jobs) bytes += 4.0 * j.np * j.n + 8.0 * j.n;
        Timed t(h, KC_PARTIAL_REDUCE, 0, bytes);
        gk::reduce_jobs(w.red_jobs, (int)h->jobs.size(), std::max({nbl, npc, npa}),
                        (int)std::max<int64_t>(d, std::max<int64_t>(3 * d, F)), w.red_tmp, st, first);
    }
    {
        Timed t(h, KC_EMBED_BWD, 0, 4.0 * M * d + 8.0 * M * d);
        if (conc) {
            wait_ev(sw, E_MAIN_END);
            gk::embed_bwd_accumulate(w.dres, G(h, tb.wte), tb.wpe >= 0 ? G(h, tb.wpe) : nullptr, B, T, d, w.emb_scratch,
                                     sw, first);
        } else {
            gpt_status s = hip_check(h, hipStreamWaitEvent(st, h->ev_join, 0), "hipStreamWaitEvent");
            if (s != GPT_OK) return s;
            gk::embed_bwd_accumulate(w.dres, G(h, tb.wte), tb.wpe >= 0 ? G(h, tb.wpe) : nullptr, B, T, d, w.emb_scratch,
                                     st, first);
        }
    }
    record(S_END, sw);
    wait_ev(st, S_END);   // every side-stream product and the embedding gradient are done
    h->micro_count += 1;
    gpt_status s = hip_check(h, hipGetLastError(), "kernel launch");
    if (s != GPT_OK) return s;
    if (h_loss) {
        s = sync_and_check(h);
        if (s != GPT_OK) return s;
        s = hip_check(h, hipMemcpy(h_loss, w.loss_last, sizeof(float), hipMemcpyDeviceToHost), "read loss");
        if (s != GPT_OK) return s;
    }
    return GPT_OK;
}

gpt_status gpt_loss_accum(gpt_handle* h, float* out) {
    if (!h || !out) return GPT_ERR_INVALID_ARGUMENT;
    gpt_status s = sync_and_check(h);
    if (s != GPT_OK) return s;
    float sum = 0.f;
    s = hip_check(h, hipMemcpy(&sum, h->ws.loss_sum, sizeof(float), hipMemcpyDeviceToHost), "read loss sum");
    if (s != GPT_OK) return s;
    *out = h->micro_count ? sum / h->micro_count : 0.f;
    return GPT_OK;
}

gpt_status gpt_generate(gpt_handle* h, const int32_t* prompt, int32_t B, int32_t T0, int32_t n_new,
                        float temperature, int32_t top_k, uint64_t seed, int32_t* out, float* logits_out) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    const gpt_config& c = h->cfg;
    if (!prompt || !out) return fail(h, GPT_ERR_INVALID_ARGUMENT, "null prompt or output buffer");
    if (B < 1 || B > c.max_batch) return fail(h, GPT_ERR_INVALID_ARGUMENT, "B must be in [1, max_batch]");
    if (T0 < 1 || n_new < 0 || (int64_t)T0 + n_new > c.block_size)
        return fail(h, GPT_ERR_INVALID_ARGUMENT, "need T0 >= 1, n_new >= 0 and T0 + n_new <= block_size");
    if (!(temperature >= 0.f) || !std::isfinite(temperature) || top_k < 0)
        return fail(h, GPT_ERR_INVALID_ARGUMENT, "temperature must be finite and >= 0, top_k >= 0");
    Ws& w = h->ws;
    const Table& tb = h->tb;
    hipStream_t st = h->stream;
    const int d = c.n_embd, F = c.mlp_hidden, Vp = c.padded_vocab_size, H = c.n_head, hd = d / H, L = c.n_layer;
    const int Tm = c.block_size, Ttot = T0 + n_new;
    const bool bf = c.precision == GPT_PREC_BF16, qkt = qk_transform(c);
    const size_t ab = bf ? 2 : 4;
    gpt_status s = hip_check(h, hipMemcpy2DAsync(out, sizeof(int32_t) * Ttot, prompt, sizeof(int32_t) * T0,
                                                 sizeof(int32_t) * T0, B, hipMemcpyDeviceToDevice, st),
                             "copy prompt");
    if (s != GPT_OK) return s;
    if (n_new > 0) {
        // prefill: the training forward over the prompt, then its keys and
        // values (q/k-transformed keys for rotary / QK-norm models) into the caches
        forward_pass(h, prompt, B, T0);
        for (int l = 0; l < L; ++l) {
            const void* ks = qkt ? (const char*)w.qk[l] + ab * d : (const char*)w.qkv[l] + ab * d;
            gk::cache_put(bf, ks, qkt ? 2 * d : 3 * d, w.kcache[l], B, T0, Tm, 0, d, st);
            gk::cache_put(bf, (const char*)w.qkv[l] + ab * 2 * d, 3 * d, w.vcache[l], B, T0, Tm, 0, d, st);
        }
        // logits of each sequence's last prompt position: rows b T0 + T0 - 1 of the final LayerNorm output
        {
            gk::Gemm g = mk_gemm(h, B, Vp, d, (const char*)w.lnf + ab * (size_t)(T0 - 1) * d, (int64_t)T0 * d, true,
                                 Wop(h, tb.wte), d, true, w.dec_logits, Vp, false, gk::EPI_STORE);
            run_decode_gemm(h, g);
        }
        gk::gen_sample(w.dec_logits, B, Vp, c.logit_softcap, temperature, top_k, seed, 0, out, Ttot, T0,
                       logits_out, st);
        for (int step = 1; step < n_new; ++step) {
            const int pos = T0 + step - 1;   // position of the token drawn last
            gk::gen_embed(out, Ttot, pos, P(h, tb.wte), tb.wpe >= 0 ? P(h, tb.wpe) : nullptr, w.dec_x, B, d, Vp,
                          w.err, st);
            // LayerNorm then product: fused into the skinny product's load of its
            // activations where that kernel applies, else the two kernels
            auto ln_gemm = [&](const float* x, int gi, int bi, gk::Gemm g) {
                gk::Gemm f = g;
                f.A = x;
                f.ln_g = P(h, gi);
                f.ln_b = P(h, bi);
                f.ln_eps = c.ln_eps;
                if (gk::skinny_gemm_ok(f)) {
                    Timed t(h, KC_MISC, 2.0 * g.M * g.N * g.K, 2.0 * (double)g.N * g.K + 4.0 * g.M * g.K,
                            "skinny_gemm_kernel");
                    gk::skinny_gemm(f, st);
                } else {
                    gk::layernorm_fwd(bf, x, P(h, gi), P(h, bi), (void*)g.A, w.dec_mean, w.dec_rstd, B, d, c.ln_eps,
                                      st);
                    run_decode_gemm(h, g);
                }
            };
            for (int l = 0; l < L; ++l) {
                const LayerIdx& li = tb.layers[l];
                {
                    gk::Gemm g = mk_gemm(h, B, 3 * d, d, w.dec_y, d, true, Wop(h, li.attn_w), d, true, w.dec_qkv,
                                         3 * d, bf, gk::EPI_BIAS);
                    g.bias = P(h, li.attn_b);
                    ln_gemm(w.dec_x, li.ln1_w, li.ln1_b, g);
                }
                const void* q = w.dec_qkv;
                const void* kn = (const char*)w.dec_qkv + ab * d;
                int64_t ldq = 3 * d;
                if (qkt) {
                    gk::qk_prep_fwd(bf, w.dec_qkv, w.dec_qk, w.rope_cos, w.rope_sin, B, 1, H, hd, c.qk_rmsnorm,
                                    c.pos_encoding == GPT_POS_ROPE, c.qk_norm_eps, st, pos);
                    q = w.dec_qk;
                    kn = (const char*)w.dec_qk + ab * d;
                    ldq = 2 * d;
                }
                gk::gen_attention(bf, q, ldq, kn, ldq, (const char*)w.dec_qkv + ab * 2 * d, 3 * d, w.kcache[l],
                                  w.vcache[l], w.dec_att, B, H, hd, pos, Tm, window_of(c, l), st);
                {
                    gk::Gemm g = mk_gemm(h, B, d, d, w.dec_att, d, true, Wop(h, li.proj_w), d, true, w.dec_x2, d, false,
                                         gk::EPI_BIAS_RESID);
                    g.bias = P(h, li.proj_b);
                    g.resid = w.dec_x;
                    run_decode_gemm(h, g);
                }
                {
                    gk::Gemm g = mk_gemm(h, B, F, d, w.dec_y, d, true, Wop(h, li.fc_w), d, true, w.dec_h1, F, bf,
                                         gk::EPI_BIAS_ACT);
                    g.bias = P(h, li.fc_b);
                    g.C2 = w.dec_h2;
                    ln_gemm(w.dec_x2, li.ln2_w, li.ln2_b, g);
                }
                {
                    gk::Gemm g = mk_gemm(h, B, d, F, w.dec_h2, F, true, Wop(h, li.mp_w), F, true, w.dec_x, d, false,
                                         gk::EPI_BIAS_RESID);
                    g.bias = P(h, li.mp_b);
                    g.resid = w.dec_x2;
                    run_decode_gemm(h, g);
                }
            }
            {
                // the head's activations are normalised once (its grid has Vp / 16 workgroups)
                gk::layernorm_fwd(bf, w.dec_x, P(h, tb.lnf_w), P(h, tb.lnf_b), w.dec_y, w.dec_mean, w.dec_rstd, B, d,
                                  c.ln_eps, st);
                gk::Gemm g = mk_gemm(h, B, Vp, d, w.dec_y, d, true, Wop(h, tb.wte), d, true, w.dec_logits, Vp, false,
                                     gk::EPI_STORE);
                run_decode_gemm(h, g);
            }
            gk::gen_sample(w.dec_logits, B, Vp, c.logit_softcap, temperature, top_k, seed, step, out, Ttot, pos + 1,
                           logits_out ? logits_out + (size_t)step * B * Vp : nullptr, st);
        }
    }
    s = hip_check(h, hipGetLastError(), "kernel launch");
    if (s != GPT_OK) return s;
    return sync_and_check(h);
}

// Global-norm clip, then AdamW on every tensor, or (muon non-null: learning
// rate, momentum) Muon on the blocks' hidden matrices and AdamW on the rest.
static gpt_status optimizer_step(gpt_handle* h, float lr, int32_t step, float* h_grad_norm, const float* muon) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    if (step < 1) return fail(h, GPT_ERR_INVALID_ARGUMENT, "step must be >= 1");
    if (!(lr >= 0.f) || !std::isfinite(lr)) return fail(h, GPT_ERR_INVALID_ARGUMENT, "lr must be finite and >= 0");
    if (muon && (!(muon[0] >= 0.f) || !std::isfinite(muon[0])))
        return fail(h, GPT_ERR_INVALID_ARGUMENT, "muon_lr must be finite and >= 0");
    if (muon && (!(muon[1] >= 0.f) || !(muon[1] < 1.f)))
        return fail(h, GPT_ERR_INVALID_ARGUMENT, "muon_momentum must be in [0, 1)");
    const gpt_config& c = h->cfg;
    Ws& w = h->ws;
    const Table& tb = h->tb;
    hipStream_t st = h->stream;
    const int64_t n = tb.n_total;
    const bool bf = c.precision == GPT_PREC_BF16;
    if (h->grads_dirty) {   // no micro-step since the last update: gradients are zero
        gk::fill_f32(w.grads, n, 0.f, st);
    }
    {
        Timed t(h, KC_GRAD_NORM, 0, 4.0 * n);
        gk::grad_norm(w.grads, n, w.gn_partial, w.gnorm, w.coef, w.nonfinite, w.err, c.max_grad_norm, st);
    }
    double b1 = c.beta1, b2 = c.beta2;
    float rbc1 = (float)(1.0 / (1.0 - std::pow(b1, step)));
    float rbc2 = (float)(1.0 / (1.0 - std::pow(b2, step)));
    if (!muon) {
        Timed t(h, KC_ADAMW, 0, 28.0 * n + 2.0 * tb.n_decay);
        gk::adamw(w.params, w.grads, w.m, w.v, w.wbf, n, tb.n_decay, w.coef, w.nonfinite, lr, c.beta1, c.beta2,
                  c.adam_eps, c.weight_decay, rbc1, rbc2, st);
    } else {
        // the hidden matrices follow the embeddings in the flat layout and end
        // the decayed range: AdamW covers [0, lo) and the undecayed tensors
        const int64_t lo = tb.t[tb.layers[0].attn_w].offset, nu = n - tb.n_decay;
        {
            Timed t(h, KC_ADAMW, 0, 28.0 * (lo + nu) + 2.0 * lo);
            gk::adamw(w.params, w.grads, w.m, w.v, w.wbf, lo, lo, w.coef, w.nonfinite, lr, c.beta1, c.beta2,
                      c.adam_eps, c.weight_decay, rbc1, rbc2, st);
            gk::adamw(w.params + tb.n_decay, w.grads + tb.n_decay, w.m + tb.n_decay, w.v + tb.n_decay, nullptr, nu, 0,
                      w.coef, w.nonfinite, lr, c.beta1, c.beta2, c.adam_eps, c.weight_decay, rbc1, rbc2, st);
        }
        // one kind of hidden matrix at a time, its n_layer matrices as one batch
        const double ab = bf ? 2 : 4;
        const int L = c.n_layer;
        for (int kind = 0; kind < 4; ++kind) {
            auto idx_of = [&](int l) {
                const LayerIdx& li = tb.layers[l];
                return kind == 0 ? li.attn_w : kind == 1 ? li.proj_w : kind == 2 ? li.fc_w : li.mp_w;
            };
            const TensorInfo& t0 = tb.t[idx_of(0)];
            const int r = (int)t0.shape[0], cc = (int)t0.shape[1], mr = std::min(r, cc), nr = std::max(r, cc);
            const int64_t mn = (int64_t)mr * nr;
            const double m2 = (double)mr * mr;
            // five iterations of three products: 2 m n m + 2 m m m + 2 m m n flops per matrix
            Timed t(h, KC_MUON, L * 5.0 * (4.0 * (double)mn * mr + 2.0 * m2 * mr),
                    L * (20.0 * mn + 5.0 * ab * (3.0 * mn + 5.0 * m2) + 12.0 * mn));
            // the layers' matrices of one kind sit at a constant stride in the flat layout
            const int64_t o0 = t0.offset, os = L > 1 ? tb.t[idx_of(1)].offset - o0 : 0;
            bool strided = true;
            for (int l = 0; l < L; ++l) strided = strided && tb.t[idx_of(l)].offset == o0 + l * os;
            const float stepsz = (float)(muon[0] * std::sqrt(std::max(1.0, (double)r / cc)));
            if (strided) {
                gk::muon_direction(w.grads + o0, w.m + o0, os, L, w.mu_u, w.mu_part, w.mu_part_stride, r, cc, muon[1],
                                   w.coef, w.nonfinite, w.mu_scale, st);
            } else {
                for (int l = 0; l < L; ++l) {
                    const int64_t ol = tb.t[idx_of(l)].offset;
                    gk::muon_direction(w.grads + ol, w.m + ol, 0, 1, w.mu_u + l * mn, w.mu_part + l * w.mu_part_stride,
                                       0, r, cc, muon[1], w.coef, w.nonfinite, w.mu_scale + l, st);
                }
            }
            char* X = (char*)gk::muon_newton_schulz(bf, w.mu_u, w.mu_scale, mr, nr, L, w.mu_x0, w.mu_x1, w.mu_a,
                                                    w.mu_aa, w.mu_b, w.splitk, w.splitk_floats, st);
            if (strided) {
                gk::muon_apply(bf, w.params + o0, bf ? (char*)w.wbf + 2 * o0 : nullptr, os, L, X, r, cc, stepsz,
                               w.nonfinite, st);
            } else {
                for (int l = 0; l < L; ++l) {
                    const int64_t ol = tb.t[idx_of(l)].offset;
                    gk::muon_apply(bf, w.params + ol, bf ? (char*)w.wbf + 2 * ol : nullptr, 0, 1,
                                   X + (size_t)ab * l * mn, r, cc, stepsz, w.nonfinite, st);
                }
            }
        }
    }
    h->grads_dirty = true;
    gpt_status s = hip_check(h, hipGetLastError(), "kernel launch");
    if (s != GPT_OK) return s;
    if (h_grad_norm) {
        // an out-of-range id (flagged on the device by a micro-step that did
        // not wait) has already made the device skip this update
        s = sync_and_check(h);
        if (s == GPT_ERR_TOKEN_RANGE) {
            (void)hipMemcpy(h_grad_norm, w.gnorm, sizeof(float), hipMemcpyDeviceToHost);
            return fail(h, GPT_ERR_TOKEN_RANGE,
                        "a token or target id is outside [0, padded_vocab_size): update skipped");
        }
        if (s != GPT_OK) return s;
        int32_t nf = 0;
        s = hip_check(h, hipMemcpy(h_grad_norm, w.gnorm, sizeof(float), hipMemcpyDeviceToHost), "read grad norm");
        if (s == GPT_OK) s = hip_check(h, hipMemcpy(&nf, w.nonfinite, sizeof(int32_t), hipMemcpyDeviceToHost), "read flag");
        if (s != GPT_OK) return s;
        if (nf) return fail(h, GPT_ERR_NONFINITE, "gradient norm is not finite: update skipped");
    }
    return GPT_OK;
}

gpt_status gpt_clip_and_adamw(gpt_handle* h, float lr, int32_t step, float* h_grad_norm) {
    return optimizer_step(h, lr, step, h_grad_norm, nullptr);
}

gpt_status gpt_clip_and_muon(gpt_handle* h, float lr, float muon_lr, float muon_momentum, int32_t step,
                             float* h_grad_norm) {
    const float mu[2] = {muon_lr, muon_momentum};
    return optimizer_step(h, lr, step, h_grad_norm, mu);
}

gpt_status gpt_num_tensors(const gpt_handle* h, int32_t* n) {
    if (!h || !n) return GPT_ERR_INVALID_ARGUMENT;
    *n = (int32_t)h->tb.t.size();
    return GPT_OK;
}

gpt_status gpt_tensor_info(const gpt_handle* h, int32_t idx, const char** name, int32_t* ndim, int64_t shape[2],
                           int32_t* decay) {
    if (!h || idx < 0 || idx >= (int32_t)h->tb.t.size()) return GPT_ERR_INVALID_ARGUMENT;
    const TensorInfo& ti = h->tb.t[idx];
    if (name) *name = ti.name.c_str();
    if (ndim) *ndim = ti.ndim;
    if (shape) { shape[0] = ti.shape[0]; shape[1] = ti.shape[1]; }
    if (decay) *decay = ti.decay;
    return GPT_OK;
}

gpt_status gpt_get_param(gpt_handle* h, int32_t idx, float* buf, int64_t count, int32_t on_dev) {
    if (check_idx(h, idx, count) != GPT_OK || !buf) return GPT_ERR_INVALID_ARGUMENT;
    return copy_tensor(h, buf, P(h, idx), count, 1, on_dev);
}
gpt_status gpt_set_param(gpt_handle* h, int32_t idx, const float* buf, int64_t count, int32_t on_dev) {
    if (check_idx(h, idx, count) != GPT_OK || !buf) return GPT_ERR_INVALID_ARGUMENT;
    gpt_status s = copy_tensor(h, P(h, idx), buf, count, 0, on_dev);
    if (s != GPT_OK) return s;
    if (h->ws.wbf && h->tb.t[idx].decay) {
        gk::f32_to_bf16((char*)h->ws.wbf + 2 * h->tb.t[idx].offset, P(h, idx), count, h->stream);
        return hip_check(h, hipStreamSynchronize(h->stream), "hipStreamSynchronize");
    }
    return GPT_OK;
}
gpt_status gpt_get_grad(gpt_handle* h, int32_t idx, float* buf, int64_t count, int32_t on_dev) {
    if (check_idx(h, idx, count) != GPT_OK || !buf) return GPT_ERR_INVALID_ARGUMENT;
    if (h->grads_dirty) gk::fill_f32(h->ws.grads, h->tb.n_total, 0.f, h->stream);
    return copy_tensor(h, buf, G(h, idx), count, 1, on_dev);
}
gpt_status gpt_set_grad(gpt_handle* h, int32_t idx, const float* buf, int64_t count, int32_t on_dev) {
    if (check_idx(h, idx, count) != GPT_OK || !buf) return GPT_ERR_INVALID_ARGUMENT;
    if (h->grads_dirty) {
        gk::fill_f32(h->ws.grads, h->tb.n_total, 0.f, h->stream);
        gk::fill_f32(h->ws.loss_sum, 1, 0.f, h->stream);
        h->grads_dirty = false;
        h->micro_count = 0;
    }
    return copy_tensor(h, G(h, idx), buf, count, 0, on_dev);
}
gpt_status gpt_get_opt_state(gpt_handle* h, int32_t idx, float* m, float* v, int64_t count, int32_t on_dev) {
    if (check_idx(h, idx, count) != GPT_OK) return GPT_ERR_INVALID_ARGUMENT;
    int64_t off = h->tb.t[idx].offset;
    if (m) { gpt_status s = copy_tensor(h, m, h->ws.m + off, count, 1, on_dev); if (s != GPT_OK) return s; }
    if (v) { gpt_status s = copy_tensor(h, v, h->ws.v + off, count, 1, on_dev); if (s != GPT_OK) return s; }
    return GPT_OK;
}
gpt_status gpt_set_opt_state(gpt_handle* h, int32_t idx, const float* m, const float* v, int64_t count, int32_t on_dev) {
    if (check_idx(h, idx, count) != GPT_OK) return GPT_ERR_INVALID_ARGUMENT;
    int64_t off = h->tb.t[idx].offset;
    if (m) { gpt_status s = copy_tensor(h, h->ws.m + off, m, count, 0, on_dev); if (s != GPT_OK) return s; }
    if (v) { gpt_status s = copy_tensor(h, h->ws.v + off, v, count, 0, on_dev); if (s != GPT_OK) return s; }
    return GPT_OK;
}

gpt_status gpt_get_row_losses(gpt_handle* h, float* buf, int64_t count, int32_t on_dev) {
    if (!h || !buf || count < 1 || count > (int64_t)h->cfg.max_batch * h->cfg.block_size)
        return GPT_ERR_INVALID_ARGUMENT;
    return copy_tensor(h, buf, h->ws.row_loss, count, 1, on_dev);
}

double gpt_lr_schedule(int32_t it, int32_t warmup, int32_t max_steps, double max_lr, double min_lr) {
    return gpth::lr_schedule(it, warmup, max_steps, max_lr, min_lr);
}

const char* gpt_status_string(gpt_status s) {
    switch (s) {
        case GPT_OK: return "ok";
        case GPT_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GPT_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case GPT_ERR_UNSUPPORTED: return "unsupported configuration or device";
        case GPT_ERR_DEVICE: return "HIP runtime error";
        case GPT_ERR_TOKEN_RANGE: return "token or target id out of range";
        case GPT_ERR_NONFINITE: return "non-finite gradient norm; update skipped";
    }
    return "unknown status";
}

const char* gpt_last_error(const gpt_handle* h) { return h ? h->last_error.c_str() : "null handle"; }

gpt_status gpt_set_kernel_timing(gpt_handle* h, int32_t mask) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    h->timing_mask = (uint32_t)mask;
    return GPT_OK;
}
gpt_status gpt_reset_kernel_timing(gpt_handle* h) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    drain_timing(h);
    for (auto& c : h->stats) c = ClassStat();
    for (auto& n : h->names) n.st = ClassStat();
    return GPT_OK;
}
gpt_status gpt_num_kernel_classes(int32_t* n) {
    if (!n) return GPT_ERR_INVALID_ARGUMENT;
    *n = KC_COUNT;
    return GPT_OK;
}
gpt_status gpt_kernel_timing(gpt_handle* h, int32_t cls, const char** name, double* total_ms, int64_t* launches,
                             double* flops, double* bytes) {
    if (!h || cls < 0 || cls >= KC_COUNT) return GPT_ERR_INVALID_ARGUMENT;
    drain_timing(h);
    if (name) *name = kc_names[cls];
    if (total_ms) *total_ms = h->stats[cls].ms;
    if (launches) *launches = h->stats[cls].launches;
    if (flops) *flops = h->stats[cls].flops;
    if (bytes) *bytes = h->stats[cls].bytes;
    return GPT_OK;
}
gpt_status gpt_set_kernel_timing_filter(gpt_handle* h, const char* kernel_name) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    h->filter = kernel_name ? kernel_name : "";
    return GPT_OK;
}
gpt_status gpt_num_kernel_names(gpt_handle* h, int32_t* n) {
    if (!h || !n) return GPT_ERR_INVALID_ARGUMENT;
    drain_timing(h);
    *n = (int32_t)h->names.size();
    return GPT_OK;
}
gpt_status gpt_kernel_name_timing(gpt_handle* h, int32_t idx, const char** name, double* total_ms, int64_t* launches,
                                  double* flops, double* bytes) {
    if (!h) return GPT_ERR_INVALID_ARGUMENT;
    drain_timing(h);
    if (idx < 0 || idx >= (int32_t)h->names.size()) return GPT_ERR_INVALID_ARGUMENT;
    const NameStat& s = h->names[idx];
    if (name) *name = s.name.c_str();
    if (total_ms) *total_ms = s.st.ms;
    if (launches) *launches = s.st.launches;
    if (flops) *flops = s.st.flops;
    if (bytes) *bytes = s.st.bytes;
    return GPT_OK;
}

// ============================================================================
// test-only kernel entry points (include/gpt_testing.h)
// ============================================================================

gpt_status gptk_gemm_force_config(int32_t cfg, int32_t splits) {
    if (cfg < -1 || cfg >= gk::gemm_mfma_num_configs() || splits < 0) return GPT_ERR_INVALID_ARGUMENT;
    gk::gemm_mfma_force(cfg, splits);
    return GPT_OK;
}
int32_t gptk_gemm_num_configs(void) { return gk::gemm_mfma_num_configs(); }

gpt_status gptk_gemm_tune(int32_t M, int32_t N, int32_t K, int32_t a_kc, int32_t b_kc, int32_t cfg, int32_t splits) {
    if (M < 1 || N < 1 || K < 1) return GPT_ERR_INVALID_ARGUMENT;
    return gk::gemm_mfma_tune(M, N, K, a_kc != 0, b_kc != 0, cfg, splits) == 0 ? GPT_OK : GPT_ERR_INVALID_ARGUMENT;
}

gpt_status gptk_gemm(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_kc, const void* B,
                     int64_t ldb, int32_t b_kc, void* C, int64_t ldc, int32_t in_bf16, int32_t c_bf16, int32_t epi,
                     int32_t act, const float* bias, const float* resid, const void* aux, void* C2,
                     float* splitk_scratch, int64_t splitk_floats, void* stream) {
    if (M < 1 || N < 1 || K < 1 || !A || !B || !C || epi < 0 || epi > 5) return GPT_ERR_INVALID_ARGUMENT;
    gk::Gemm g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.a_kc = a_kc;
    g.B = B; g.ldb = ldb; g.b_kc = b_kc;
    g.C = C; g.ldc = ldc; g.c_bf = c_bf16;
    g.C2 = C2; g.bias = bias; g.resid = resid; g.aux = aux;
    g.epi = epi; g.act = act; g.in_bf = in_bf16;
    gk::gemm(g, splitk_scratch, (size_t)splitk_floats, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

gpt_status gptk_gemm_colsum(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_kc, const void* B,
                            int64_t ldb, int32_t b_kc, void* C, int64_t ldc, int32_t in_bf16, int32_t c_bf16,
                            int32_t epi, int32_t act, const float* bias, const float* resid, const void* aux, void* C2,
                            float* colsum_out, float* partial, float* splitk_scratch, int64_t splitk_floats,
                            void* stream) {
    if (M < 1 || N < 1 || K < 1 || !A || !B || !C || !colsum_out || !partial || epi < 0 || epi > 5)
        return GPT_ERR_INVALID_ARGUMENT;
    if (epi == gk::EPI_ACCUM) return GPT_ERR_UNSUPPORTED;
    gk::Gemm g{};
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.a_kc = a_kc;
    g.B = B; g.ldb = ldb; g.b_kc = b_kc;
    g.C = C; g.ldc = ldc; g.c_bf = c_bf16;
    g.C2 = C2; g.bias = bias; g.resid = resid; g.aux = aux;
    g.epi = epi; g.act = act; g.in_bf = in_bf16;
    hipStream_t s = (hipStream_t)stream;
    const gk::GemmPlan p = gk::gemm_plan(g, (size_t)splitk_floats);
    if (p.bm > 0) {
        g.cpart = partial;
        gk::gemm_main(g, p, splitk_scratch, s);
        gk::gemm_finish(g, p, splitk_scratch, s);
        const int np = (M + p.bm - 1) / p.bm;
        gk::reduce_rows(partial, np, N, colsum_out, partial + (size_t)np * N, s);
    } else {
        gk::gemm_main(g, p, splitk_scratch, s);
        gk::gemm_finish(g, p, splitk_scratch, s);
        const bool out_bf = epi != gk::EPI_BIAS_RESID && c_bf16 != 0;   // the residual epilogue stores fp32
        gk::colsum(out_bf, C, ldc, M, N, colsum_out, partial, s);
    }
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

gpt_status gptk_attention(int32_t backward, int32_t B, int32_t T, int32_t H, int32_t hd, int32_t window,
                          const void* q, const void* k, const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                          void* o, int64_t ldo, float* lse, const void* dO, int64_t lddo, float* D, void* dq, void* dk,
                          void* dv, int64_t ldd, int32_t bf16, void* stream) {
    if (B < 1 || T < 1 || H < 1 || (hd != 16 && hd != 32 && hd != 64 && hd != 128)) return GPT_ERR_INVALID_ARGUMENT;
    gk::Attn a{};
    a.B = B; a.T = T; a.H = H; a.hd = hd; a.window = window;
    a.q = q; a.k = k; a.v = v; a.ldq = ldq; a.ldk = ldk; a.ldv = ldv;
    a.o = o; a.ldo = ldo; a.lse = lse; a.dO = dO; a.lddo = lddo; a.D = D; a.Dout = D;
    a.dq = dq; a.dk = dk; a.dv = dv; a.ldd = ldd; a.bf = bf16;
    hipStream_t s = (hipStream_t)stream;
    if (backward) {
        gk::attention_bwd(a, s);
    } else {
        gk::attention_fwd(a, s);
    }
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

int64_t gptk_attention_colsum_partial_floats(int32_t B, int32_t T, int32_t H, int32_t hd) {
    if (B < 1 || T < 1 || H < 1 || hd < 1) return 0;
    const int64_t n = 3LL * H * hd;
    const int64_t npa = (int64_t)B * ((T + 127) / 128);
    const int64_t fused = npa * n + (npa + 63) / 64 * n;
    return std::max<int64_t>(fused, gptk_colsum_partial_floats(B * T, (int32_t)n));
}

gpt_status gptk_attention_bwd_colsum(int32_t B, int32_t T, int32_t H, int32_t hd, int32_t window, const void* q,
                                     const void* k, const void* v, int64_t ldq, int64_t ldk, int64_t ldv, const void* o,
                                     int64_t ldo, const float* lse, const void* dO, int64_t lddo, float* D, void* dqkv,
                                     int32_t bf16, float* colsum_out, float* partial, void* stream) {
    if (B < 1 || T < 1 || H < 1 || (hd != 16 && hd != 32 && hd != 64 && hd != 128) || !dqkv || !colsum_out || !partial)
        return GPT_ERR_INVALID_ARGUMENT;
    const int64_t d = (int64_t)H * hd;
    const size_t es = bf16 ? 2 : 4;
    gk::Attn a{};
    a.B = B; a.T = T; a.H = H; a.hd = hd; a.window = window;
    a.q = q; a.k = k; a.v = v; a.ldq = ldq; a.ldk = ldk; a.ldv = ldv;
    a.o = (void*)o; a.ldo = ldo; a.lse = (float*)lse; a.dO = dO; a.lddo = lddo; a.D = D; a.Dout = D;
    a.dq = dqkv; a.dk = (char*)dqkv + es * d; a.dv = (char*)dqkv + es * 2 * d; a.ldd = 3 * d; a.bf = bf16;
    a.cpart = partial;
    hipStream_t s = (hipStream_t)stream;
    if (gk::attention_bwd(a, s)) {
        const int npa = B * ((T + 127) / 128);
        gk::reduce_rows(partial, npa, (int)(3 * d), colsum_out, partial + (size_t)npa * 3 * d, s);
    } else {
        gk::colsum(bf16 != 0, dqkv, 3 * d, B * T, (int)(3 * d), colsum_out, partial, s);
    }
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

gpt_status gptk_layernorm(int32_t backward, int32_t M, int32_t d, float eps, const float* x, const float* g,
                          const float* b, void* y, float* mean, float* rstd, const float* dy, float* dres,
                          void* dres_lp, int32_t overwrite, float* dg, float* db, float* dcol, float* partial,
                          int32_t bf16, void* stream) {
    if (M < 1 || d < 4 || d % 4 || d > 2048) return GPT_ERR_INVALID_ARGUMENT;
    hipStream_t s = (hipStream_t)stream;
    if (backward)
        gk::layernorm_bwd(bf16, dy, x, mean, rstd, g, dres, dres_lp, overwrite, dg, db, dcol, partial, M, d, s);
    else gk::layernorm_fwd(bf16, x, g, b, y, mean, rstd, M, d, eps, s);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

int64_t gptk_layernorm_partial_floats(int32_t M, int32_t d) { return (int64_t)gk::layernorm_bwd_partial_floats(M, d); }

gpt_status gptk_layernorm_bwd_noalloc(int32_t M, int32_t d, const float* x, const float* g, const float* mean,
                                      const float* rstd, const float* dy, float* dres, void* dres_lp,
                                      int32_t overwrite, float* dg, float* db, float* dcol, int32_t bf16,
                                      void* stream) {
    if (M < 1 || d < 4 || d % 4 || d > 2048 || !x || !g || !mean || !rstd || !dy || !dres || !dg || !db)
        return GPT_ERR_INVALID_ARGUMENT;
    const int r = gk::layernorm_bwd_static(bf16, dy, x, mean, rstd, g, dres, dres_lp, overwrite, dg, db, dcol, M, d,
                                           (hipStream_t)stream);
    if (r == -1) return GPT_ERR_INVALID_ARGUMENT;
    if (r != 0) return GPT_ERR_DEVICE;
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

int64_t gptk_layernorm_noalloc_max_floats(void) { return (int64_t)gk::layernorm_bwd_static_capacity_floats(); }

gpt_status gptk_cross_entropy(int32_t M, int32_t Vp, void* z, const int32_t* y, float* row_loss, float gscale,
                              float cap, int32_t* err, int32_t bf16, void* stream) {
    if (M < 1 || Vp < 1) return GPT_ERR_INVALID_ARGUMENT;
    gk::cross_entropy(bf16, z, y, row_loss, M, Vp, gscale, cap, err, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

gpt_status gptk_qk_prep(int32_t backward, int32_t M, int32_t T, int32_t H, int32_t hd, const void* qkv, void* out,
                        float* tables, double base, int32_t norm, int32_t rope, float eps, int32_t bf16,
                        void* stream) {
    if (M < 1 || T < 1 || H < 1 || hd < 2 || hd % 2 || hd > 128 || !qkv || !out || !tables || !(base > 0.0))
        return GPT_ERR_INVALID_ARGUMENT;
    const hipStream_t s = (hipStream_t)stream;
    float* cos_t = tables;
    float* sin_t = tables + (size_t)T * (hd / 2);
    gk::rope_tables(cos_t, sin_t, T, hd, base, s);
    if (backward)
        gk::qk_prep_bwd(bf16, qkv, out, cos_t, sin_t, M, T, H, hd, norm, rope, eps, s);
    else
        gk::qk_prep_fwd(bf16, qkv, out, cos_t, sin_t, M, T, H, hd, norm, rope, eps, s, 0);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

int64_t gptk_embed_bwd_scratch_bytes(int32_t M, int32_t d) { return (int64_t)gk::embed_bwd_scratch_bytes(M, d); }

int64_t gptk_gemm_fp8_scratch_bytes(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || N < 1 || K < 1) return 0;
    return (((int64_t)M * K + 255) / 256 + ((int64_t)N * K + 255) / 256) * 256 + 256 + 2048 * 4;
}

gpt_status gptk_gemm_fp8(int32_t M, int32_t N, int32_t K, const void* A, const void* B, void* C, void* scratch,
                         int64_t scratch_bytes, void* stream) {
    if (M < 1 || N < 1 || K < 128 || K % 128 || N % 8 || !A || !B || !C || !scratch ||
        scratch_bytes < gptk_gemm_fp8_scratch_bytes(M, N, K) || (uintptr_t)scratch % 256 || (uintptr_t)A % 16 ||
        (uintptr_t)B % 16 || (uintptr_t)C % 16)
        return GPT_ERR_INVALID_ARGUMENT;
    char* p = (char*)scratch;
    uint8_t* aq = (uint8_t*)p;
    p += ((int64_t)M * K + 255) / 256 * 256;
    uint8_t* bq = (uint8_t*)p;
    p += ((int64_t)N * K + 255) / 256 * 256;
    float* sc = (float*)p;
    float* part = sc + 64;
    hipStream_t s = (hipStream_t)stream;
    gk::quantize_e4m3(A, (int64_t)M * K, aq, sc + 2, sc, part, s);
    gk::quantize_e4m3(B, (int64_t)N * K, bq, sc + 3, sc + 1, part + 1024, s);
    gk::gemm_f8(M, N, K, aq, K, bq, K, C, N, sc, s);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

// scratch layout of gptk_muon_orthogonalize: buffer and direction (fp32, r c
// each), two iterates (m n), A, A A, a I + b A + c A A (m m), tile sums, the
// unit clip coefficient and the normalisation (two floats), and a cleared skip flag
static int64_t muon_test_layout(int32_t r, int32_t c, int32_t bf16, int64_t off[10]) {
    const int64_t rc = (int64_t)r * c, m = std::min(r, c), ab = bf16 ? 2 : 4;
    const int64_t sz[10] = {4 * rc, 4 * rc, ab * rc, ab * rc, ab * m * m, ab * m * m, ab * m * m,
                            4 * gk::muon_part_floats(r, c), 8, 4};
    int64_t o = 0;
    for (int i = 0; i < 10; ++i) {
        off[i] = o;
        o += (sz[i] + 255) / 256 * 256;
    }
    return o;
}

int64_t gptk_muon_scratch_bytes(int32_t r, int32_t c, int32_t bf16) {
    if (r < 1 || c < 1) return 0;
    int64_t off[10];
    return muon_test_layout(r, c, bf16, off);
}

gpt_status gptk_muon_orthogonalize(int32_t r, int32_t c, const float* G, float* O, int32_t bf16, void* scratch,
                                   int64_t scratch_bytes, void* stream) {
    if (r < 1 || c < 1 || !G || !O || !scratch || (uintptr_t)scratch % 256 ||
        scratch_bytes < gptk_muon_scratch_bytes(r, c, bf16))
        return GPT_ERR_INVALID_ARGUMENT;
    int64_t off[10];
    (void)muon_test_layout(r, c, bf16, off);
    char* p = (char*)scratch;
    auto at = [&](int i) { return (void*)(p + off[i]); };
    hipStream_t s = (hipStream_t)stream;
    const int m = std::min(r, c), n = std::max(r, c);
    float* one = (float*)at(8);
    int32_t* skip = (int32_t*)at(9);
    gk::fill_f32((float*)at(0), (int64_t)r * c, 0.f, s);
    gk::fill_f32(one, 1, 1.f, s);
    gk::fill_i32(skip, 1, 0, s);
    gk::fill_f32(O, (int64_t)r * c, 0.f, s);
    // momentum 0 from a zero buffer: the direction is G itself
    gk::muon_direction(G, (float*)at(0), 0, 1, (float*)at(1), (float*)at(7), 0, r, c, 0.f, one, skip, one + 1, s);
    void* X = gk::muon_newton_schulz(bf16 != 0, (float*)at(1), one + 1, m, n, 1, at(2), at(3), at(4), at(5), at(6),
                                     nullptr, 0, s);
    gk::muon_apply(bf16 != 0, O, nullptr, 0, 1, X, r, c, -1.f, skip, s);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

gpt_status gptk_embed_bwd(const int32_t* tok, const float* dx, float* dwte, float* dwpe, int32_t B, int32_t T,
                          int32_t d, int32_t Vp, void* scratch, void* stream) {
    if (B < 1 || T < 1 || (int64_t)B * T > 32768 || d % 4 || Vp > 131071) return GPT_ERR_INVALID_ARGUMENT;
    gk::embed_bwd(tok, dx, dwte, dwpe, B, T, d, Vp, scratch, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

gpt_status gptk_colsum(int32_t M, int32_t N, const void* Y, int64_t ld, int32_t bf16, float* out, float* partial,
                       void* stream) {
    if (M < 1 || N < 1) return GPT_ERR_INVALID_ARGUMENT;
    gk::colsum(bf16, Y, ld, M, N, out, partial, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

int64_t gptk_colsum_partial_floats(int32_t M, int32_t N) { return (int64_t)gk::colsum_partial_floats(M, N); }

gpt_status gptk_sample(float* logits, int32_t B, int32_t Vp, float cap, float temperature, int32_t top_k, uint64_t seed,
                       int32_t step, int32_t* tokens, void* stream) {
    if (B < 1 || Vp < 1 || !logits || !tokens || !(temperature >= 0.f) || !(cap >= 0.f))
        return GPT_ERR_INVALID_ARGUMENT;
    gk::gen_sample(logits, B, Vp, cap, temperature, top_k, seed, step, tokens, 1, 0, nullptr, (hipStream_t)stream);
    return hipGetLastError() == hipSuccess ? GPT_OK : GPT_ERR_DEVICE;
}

}  // extern "C"
