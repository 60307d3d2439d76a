// Host-only checks of the library's model description (configuration
// validation and defaults, parameter table, learning-rate schedule), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py. Prints "ok" and exits 0 when every check holds.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "../../transformer_lm_step_gpt_amd/csrc/host_model.h"

static int fails = 0;
#define CHECK(cond, ...)                                              \
    do {                                                              \
        if (!(cond)) {                                                \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);          \
            std::printf(__VA_ARGS__);                                 \
            std::printf("\n");                                        \
            ++fails;                                                  \
        }                                                             \
    } while (0)

// every tensor 64-aligned, inside its region (decayed prefix, then the rest),
// no two overlapping, and the totals consistent
static void check_table(const gpt_config& c, const gpth::Table& tb) {
    std::vector<std::pair<int64_t, int64_t>> spans;
    int64_t numel = 0;
    for (const auto& t : tb.t) {
        CHECK(t.offset % 64 == 0, "%s offset %lld not 64-aligned", t.name.c_str(), (long long)t.offset);
        CHECK(t.numel == (t.ndim == 2 ? t.shape[0] * t.shape[1] : t.shape[0]), "%s numel", t.name.c_str());
        CHECK(t.decay == (t.ndim == 2), "%s decay flag", t.name.c_str());
        if (t.decay) CHECK(t.offset + t.numel <= tb.n_decay, "%s outside the decayed prefix", t.name.c_str());
        else CHECK(t.offset >= tb.n_decay && t.offset + t.numel <= tb.n_total, "%s outside its region", t.name.c_str());
        spans.push_back({t.offset, t.offset + t.numel});
        numel += t.numel;
    }
    for (size_t i = 0; i < spans.size(); ++i)
        for (size_t j = i + 1; j < spans.size(); ++j)
            CHECK(spans[i].second <= spans[j].first || spans[j].second <= spans[i].first, "tensors %zu and %zu overlap",
                  i, j);
    CHECK((int)tb.layers.size() == c.n_layer, "layer count");
    CHECK(tb.n_total >= numel && tb.n_total % 64 == 0 && tb.n_decay % 64 == 0, "totals");
    CHECK((tb.wpe >= 0) == (c.pos_encoding == GPT_POS_LEARNED), "wpe present iff learned positions");
}

// xorshift64 for the configuration fuzz
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return rng_state;
}
static int pick(std::initializer_list<int> v) { return *(v.begin() + next_u64() % v.size()); }

int main() {
    // defaults: the GPT-2 124M configuration; parameter counts the Lecture prints
    gpt_config c;
    gpth::config_defaults(&c);
    std::string why;
    CHECK(gpth::validate_config(&c, &why) == GPT_OK, "defaults rejected: %s", why.c_str());
    gpth::Table tb = gpth::build_table(c);
    int64_t numel = 0, nd = 0, nu = 0, small = 0;
    for (const auto& t : tb.t) {
        numel += t.numel;
        (t.decay ? nd : nu) += 1;
        if (!t.decay) small += t.numel;
    }
    CHECK(numel == 124475904, "124M parameter count %lld", (long long)numel);
    CHECK(nd == 50 && nu == 98, "decayed / undecayed tensors %lld / %lld", (long long)nd, (long long)nu);
    CHECK(small == 121344, "undecayed numbers %lld", (long long)small);
    check_table(c, tb);

    // rejected configurations and their statuses
    struct Case {
        const char* what;
        void (*mutate)(gpt_config*);
        gpt_status want;
    };
    const Case cases[] = {
        {"no layers", [](gpt_config* x) { x->n_layer = 0; }, GPT_ERR_INVALID_ARGUMENT},
        {"n_embd not a multiple of n_head", [](gpt_config* x) { x->n_head = 7; }, GPT_ERR_INVALID_ARGUMENT},
        {"padded vocab below vocab", [](gpt_config* x) { x->padded_vocab_size = 50000; }, GPT_ERR_INVALID_ARGUMENT},
        {"unknown precision", [](gpt_config* x) { x->precision = 7; }, GPT_ERR_INVALID_ARGUMENT},
        {"unknown position encoding", [](gpt_config* x) { x->pos_encoding = -1; }, GPT_ERR_INVALID_ARGUMENT},
        {"unknown activation", [](gpt_config* x) { x->mlp_act = 9; }, GPT_ERR_INVALID_ARGUMENT},
        {"negative window", [](gpt_config* x) { x->window_even = -1; }, GPT_ERR_INVALID_ARGUMENT},
        {"NaN softcap", [](gpt_config* x) { x->logit_softcap = std::nanf(""); }, GPT_ERR_INVALID_ARGUMENT},
        {"zero LayerNorm epsilon", [](gpt_config* x) { x->ln_eps = 0.f; }, GPT_ERR_INVALID_ARGUMENT},
        {"head dim 96", [](gpt_config* x) { x->n_head = 8; }, GPT_ERR_UNSUPPORTED},
        {"too many rows", [](gpt_config* x) { x->max_batch = 64; }, GPT_ERR_UNSUPPORTED},
        {"vocabulary too large", [](gpt_config* x) { x->vocab_size = x->padded_vocab_size = 200000; }, GPT_ERR_UNSUPPORTED},
        {"head_fp8 not a flag", [](gpt_config* x) { x->head_fp8 = 2; }, GPT_ERR_INVALID_ARGUMENT},
        {"FP8 head on fp32", [](gpt_config* x) { x->head_fp8 = 1; x->precision = GPT_PREC_FP32; }, GPT_ERR_UNSUPPORTED},
    };
    for (const Case& k : cases) {
        gpt_config x = c;
        k.mutate(&x);
        why.clear();
        const gpt_status s = gpth::validate_config(&x, &why);
        CHECK(s == k.want, "%s: status %d, expected %d", k.what, (int)s, (int)k.want);
        CHECK(!why.empty(), "%s: no reason given", k.what);
    }
    CHECK(gpth::validate_config(nullptr, &why) == GPT_ERR_INVALID_ARGUMENT, "null config");

    // fuzz: random configurations around the supported ranges; every accepted one
    // must give a consistent table
    int accepted = 0;
    for (int i = 0; i < 20000; ++i) {
        gpt_config x = c;
        x.n_layer = pick({-1, 0, 1, 2, 3, 6, 12});
        x.n_head = pick({0, 1, 2, 3, 4, 6, 8, 12});
        x.n_embd = pick({0, 8, 32, 48, 64, 96, 128, 256, 384, 768, 1536, 4096});
        x.mlp_hidden = pick({0, 4, 64, 256, 1536, 3072});
        x.block_size = pick({0, 1, 7, 64, 256, 1024, 2048});
        x.vocab_size = pick({0, 1, 65, 50257});
        x.padded_vocab_size = x.vocab_size + pick({-1, 0, 3, 47});
        x.max_batch = pick({0, 1, 4, 16, 64});
        x.precision = pick({0, 1, 2});
        x.pos_encoding = pick({0, 1, 2});
        x.mlp_act = pick({0, 1, 5});
        x.head_fp8 = pick({0, 1});
        x.window_even = pick({-3, 0, 5, 256});
        if (gpth::validate_config(&x, &why) == GPT_OK) {
            ++accepted;
            check_table(x, gpth::build_table(x));
        }
    }
    CHECK(accepted > 50, "fuzz accepted only %d configurations", accepted);

    // learning-rate schedule: warmup (it + 1) / warmup, cosine to min_lr, min_lr after
    CHECK(std::fabs(gpth::lr_schedule(0, 715, 19073, 6e-4, 6e-5) - 6e-4 / 715) < 1e-18, "first warmup step");
    CHECK(std::fabs(gpth::lr_schedule(714, 715, 19073, 6e-4, 6e-5) - 6e-4) < 1e-18, "last warmup step");
    CHECK(std::fabs(gpth::lr_schedule(715, 715, 19073, 6e-4, 6e-5) - 6e-4) < 1e-15, "start of the decay");
    CHECK(std::fabs(gpth::lr_schedule(19073, 715, 19073, 6e-4, 6e-5) - 6e-5) < 1e-15, "end of the decay");
    CHECK(gpth::lr_schedule(30000, 715, 19073, 6e-4, 6e-5) == 6e-5, "after the decay");
    double prev = 1.0;
    for (int it = 715; it <= 19073; it += 97) {
        const double v = gpth::lr_schedule(it, 715, 19073, 6e-4, 6e-5);
        CHECK(v <= prev && v >= 6e-5 - 1e-18, "decay not monotone at %d", it);
        prev = v;
    }
    std::printf("%s\n", fails ? "FAILED" : "ok");
    return fails ? 1 : 0;
}
