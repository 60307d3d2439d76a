// Host-side model description (see host_model.h): validation, defaults,
// parameter table, learning-rate schedule.
#include "host_model.h"

#include <cmath>
#include <cstring>

namespace gpth {

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

Table build_table(const gpt_config& c) {
    Table tb;
    auto add = [&](const std::string& n, int64_t r, int64_t cols, int init) {
        TensorInfo ti;
        ti.name = n;
        ti.ndim = cols > 0 ? 2 : 1;
        ti.shape[0] = r;
        ti.shape[1] = cols > 0 ? cols : 0;
        ti.numel = cols > 0 ? r * cols : r;
        ti.decay = cols > 0 ? 1 : 0;
        ti.init = init;
        ti.offset = 0;
        tb.t.push_back(ti);
        return (int)tb.t.size() - 1;
    };
    const int64_t d = c.n_embd, F = c.mlp_hidden;
    tb.wte = add("wte", c.padded_vocab_size, d, INIT_NORMAL);
    if (c.pos_encoding == GPT_POS_LEARNED) tb.wpe = add("wpe", c.block_size, d, INIT_NORMAL);
    for (int l = 0; l < c.n_layer; ++l) {
        std::string p = "h." + std::to_string(l) + ".";
        LayerIdx li;
        li.ln1_w = add(p + "ln_1.weight", d, 0, INIT_ONE);
        li.ln1_b = add(p + "ln_1.bias", d, 0, INIT_ZERO);
        li.attn_w = add(p + "attn.c_attn.weight", 3 * d, d, INIT_NORMAL);
        li.attn_b = add(p + "attn.c_attn.bias", 3 * d, 0, INIT_ZERO);
        li.proj_w = add(p + "attn.c_proj.weight", d, d, INIT_PROJ);
        li.proj_b = add(p + "attn.c_proj.bias", d, 0, INIT_ZERO);
        li.ln2_w = add(p + "ln_2.weight", d, 0, INIT_ONE);
        li.ln2_b = add(p + "ln_2.bias", d, 0, INIT_ZERO);
        li.fc_w = add(p + "mlp.c_fc.weight", F, d, INIT_NORMAL);
        li.fc_b = add(p + "mlp.c_fc.bias", F, 0, INIT_ZERO);
        li.mp_w = add(p + "mlp.c_proj.weight", d, F, INIT_PROJ);
        li.mp_b = add(p + "mlp.c_proj.bias", d, 0, INIT_ZERO);
        tb.layers.push_back(li);
    }
    tb.lnf_w = add("ln_f.weight", d, 0, INIT_ONE);
    tb.lnf_b = add("ln_f.bias", d, 0, INIT_ZERO);
    // flat layout: every decayed (2-D) tensor first, then the rest; 64-element alignment
    int64_t off = 0;
    for (auto& ti : tb.t)
        if (ti.decay) { ti.offset = off; off = align_up(off + ti.numel, 64); }
    tb.n_decay = off;
    for (auto& ti : tb.t)
        if (!ti.decay) { ti.offset = off; off = align_up(off + ti.numel, 64); }
    tb.n_total = off;
    return tb;
}

gpt_status validate_config(const gpt_config* c, std::string* why) {
    auto bad = [&](gpt_status s, const char* msg) { if (why) *why = msg; return s; };
    if (!c) return bad(GPT_ERR_INVALID_ARGUMENT, "null config");
    if (c->n_layer < 1 || c->n_head < 1 || c->n_embd < 1 || c->mlp_hidden < 1 || c->block_size < 1 ||
        c->vocab_size < 1 || c->padded_vocab_size < 1 || c->max_batch < 1)
        return bad(GPT_ERR_INVALID_ARGUMENT, "sizes must be positive");
    if (c->n_embd % c->n_head) return bad(GPT_ERR_INVALID_ARGUMENT, "n_embd not divisible by n_head");
    if (c->padded_vocab_size < c->vocab_size) return bad(GPT_ERR_INVALID_ARGUMENT, "padded_vocab_size < vocab_size");
    if (c->precision != GPT_PREC_FP32 && c->precision != GPT_PREC_BF16)
        return bad(GPT_ERR_INVALID_ARGUMENT, "unknown precision");
    if (c->pos_encoding != GPT_POS_LEARNED && c->pos_encoding != GPT_POS_ROPE)
        return bad(GPT_ERR_INVALID_ARGUMENT, "unknown pos_encoding");
    if (c->mlp_act != GPT_ACT_GELU_TANH && c->mlp_act != GPT_ACT_RELU2)
        return bad(GPT_ERR_INVALID_ARGUMENT, "unknown mlp_act");
    if (c->window_even < 0 || c->window_odd < 0) return bad(GPT_ERR_INVALID_ARGUMENT, "negative window");
    if (c->logit_softcap < 0.f || !std::isfinite(c->logit_softcap)) return bad(GPT_ERR_INVALID_ARGUMENT, "bad softcap");
    if (!(c->ln_eps > 0.f) || !(c->adam_eps >= 0.f) || !(c->max_grad_norm > 0.f) || !(c->init_std >= 0.0))
        return bad(GPT_ERR_INVALID_ARGUMENT, "bad epsilon, max_grad_norm or init_std");
    const int hd = c->n_embd / c->n_head;
    if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return bad(GPT_ERR_UNSUPPORTED, "head dim must be 16, 32, 64 or 128");
    if (c->n_embd % 8 || c->mlp_hidden % 8) return bad(GPT_ERR_UNSUPPORTED, "n_embd and mlp_hidden must be multiples of 8");
    if (c->n_embd > 2048) return bad(GPT_ERR_UNSUPPORTED, "n_embd > 2048");
    if ((int64_t)c->max_batch * c->block_size > 32768) return bad(GPT_ERR_UNSUPPORTED, "max_batch * block_size > 32768");
    if (c->padded_vocab_size > 131071) return bad(GPT_ERR_UNSUPPORTED, "padded_vocab_size > 131071");
    if (c->head_fp8 != 0 && c->head_fp8 != 1) return bad(GPT_ERR_INVALID_ARGUMENT, "head_fp8 must be 0 or 1");
    if (c->head_fp8 && (c->precision != GPT_PREC_BF16 || c->n_embd % 128))
        return bad(GPT_ERR_UNSUPPORTED, "head_fp8 needs bf16 precision and n_embd % 128 == 0");
    return GPT_OK;
}


void config_defaults(gpt_config* c) {
    std::memset(c, 0, sizeof(*c));
    c->n_layer = 12; c->n_head = 12; c->n_embd = 768; c->mlp_hidden = 3072;
    c->block_size = 1024; c->vocab_size = 50257; c->padded_vocab_size = 50304; c->max_batch = 16;
    c->precision = GPT_PREC_BF16; c->pos_encoding = GPT_POS_LEARNED; c->mlp_act = GPT_ACT_GELU_TANH;
    c->ln_eps = 1e-5f; c->qk_norm_eps = 1e-6f; c->rope_base = 10000.f; c->logit_softcap = 0.f;
    c->beta1 = 0.9f; c->beta2 = 0.95f; c->adam_eps = 1e-8f; c->weight_decay = 0.1f; c->max_grad_norm = 1.0f;
    c->init_std = 0.02;
}

double lr_schedule(int32_t it, int32_t warmup, int32_t max_steps, double max_lr, double min_lr) {
    if (it < warmup) return max_lr * (it + 1) / warmup;
    if (it > max_steps) return min_lr;
    double ratio = (double)(it - warmup) / (double)(max_steps - warmup);
    double coeff = 0.5 * (1.0 + std::cos(M_PI * ratio));
    return min_lr + coeff * (max_lr - min_lr);
}

}  // namespace gpth
