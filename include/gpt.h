/*
 * gpt.h -- C ABI of the GPT-2 training-step library for AMD Instinct MI355X
 * (gfx950). One handle holds one model (parameters, gradients, AdamW moments,
 * activations) inside a caller-provided device workspace and runs its kernels
 * on a caller-provided HIP stream.
 *
 * The calls reproduce the user-level operations of the training loop the
 * source pages describe:
 *   model(x, targets=y) -> loss, loss.backward()   -> gpt_forward_backward
 *   clip_grad_norm_(params, 1.0); optimizer.step(); zero_grad()
 *                                                  -> gpt_clip_and_adamw
 *   get_lr(it)                                     -> gpt_lr_schedule
 *   model.parameters() / .grad                     -> gpt_get_param / gpt_get_grad
 * ("NanoGPT Speedrun baseline" (cruxr.ai), "Configuración del Entrenamiento";
 *  "Zero to Hero, lecture 9: reproducing GPT-2 (124M)" (ai.flicky.cc),
 *  "Оптимизатор, клиппинг, расписание" and "Накопление градиентов").
 *
 * Conventions
 *   - Every call returns a gpt_status; GPT_OK is 0, errors are negative.
 *   - Device pointers are plain HIP device addresses; "stream" arguments are
 *     hipStream_t values passed as void*.
 *   - The caller owns every buffer it passes; the library never frees them.
 *   - Calls on one handle are not thread-safe. Calls are asynchronous on the
 *     handle's stream unless stated otherwise.
 *   - Integer token ids are int32, row-major [B, T].
 */
#ifndef GPT_MI355X_H
#define GPT_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gpt_status {
    GPT_OK = 0,
    GPT_ERR_INVALID_ARGUMENT = -1,   /* null pointer, shape out of range, bad index */
    GPT_ERR_WORKSPACE_TOO_SMALL = -2,
    GPT_ERR_UNSUPPORTED = -3,        /* configuration the kernels do not implement */
    GPT_ERR_DEVICE = -4,             /* a HIP runtime call failed */
    GPT_ERR_TOKEN_RANGE = -5,        /* a token or target id outside [0, padded_vocab) */
    GPT_ERR_NONFINITE = -6           /* non-finite gradient norm: update skipped */
} gpt_status;

enum { GPT_PREC_FP32 = 0, GPT_PREC_BF16 = 1 };
enum { GPT_POS_LEARNED = 0, GPT_POS_ROPE = 1 };
enum { GPT_ACT_GELU_TANH = 0, GPT_ACT_RELU2 = 1 };

/*
 * Model and optimiser configuration. Shape fields follow the lecture's
 * GPTConfig (block_size, vocab_size, n_layer, n_head, n_embd; "Раздел 1 /
 * Архитектура"); mlp_hidden is the MLP width (4 n_embd for GPT-2);
 * padded_vocab_size >= vocab_size is the number of wte rows and lm_head
 * columns (50304 for GPT-2, "Раздел 2. Сделаем быстро": a vocabulary size
 * divisible by 128; the extra rows are ordinary, trainable classes).
 * max_batch bounds B in gpt_forward_backward and sizes the activations.
 *
 * The speedrun-block fields implement the Modded-NanoGPT README's technique
 * list: rotary positions instead of wpe (pos_encoding), parameter-free RMS
 * normalisation of q and k per head (qk_rmsnorm), ReLU^2 MLP (mlp_act),
 * sliding-window causal attention with window_even/window_odd keys on
 * even/odd layers (0 = plain causal), a tanh logit softcap
 * (logit_softcap * tanh(z / logit_softcap); 0 = off) and zero-initialised
 * output projections (zero_init_proj). The same list names an FP8 matmul for
 * the output head: head_fp8 computes z = LN_f(x) wte^T from e4m3 copies of
 * both operands (the softcap, when set, applies to that z).
 */
typedef struct gpt_config {
    int32_t n_layer;
    int32_t n_head;
    int32_t n_embd;
    int32_t mlp_hidden;
    int32_t block_size;
    int32_t vocab_size;
    int32_t padded_vocab_size;
    int32_t max_batch;
    int32_t precision;        /* GPT_PREC_FP32: all-fp32 kernels;
                                 GPT_PREC_BF16: bf16 matmul operands and stored
                                 activations, fp32 accumulation, fp32 residual
                                 stream, norms, softmax, loss, grads, master weights */
    int32_t pos_encoding;     /* GPT_POS_LEARNED or GPT_POS_ROPE */
    int32_t qk_rmsnorm;       /* 0 or 1 */
    int32_t mlp_act;          /* GPT_ACT_GELU_TANH or GPT_ACT_RELU2 */
    int32_t window_even;      /* keys visible to query i: j <= i and i - j < W (W > 0) */
    int32_t window_odd;
    int32_t zero_init_proj;   /* 0 or 1 */
    int32_t head_fp8;         /* 0 or 1: the tied head's forward product on e4m3
                                 operands with per-tensor scales 448 / max|t| (bf16
                                 precision, n_embd % 128 == 0); the backward uses the
                                 bf16 operands */
    float ln_eps;             /* LayerNorm epsilon, biased variance (1e-5) */
    float qk_norm_eps;        /* 1e-6 */
    float rope_base;          /* 10000 */
    float logit_softcap;      /* 0 = off */
    float beta1;              /* 0.9  */
    float beta2;              /* 0.95 */
    float adam_eps;           /* 1e-8 */
    float weight_decay;       /* 0.1, applied to every 2-D tensor */
    float max_grad_norm;      /* 1.0 */
    int32_t reserved1;
    double init_std;          /* 0.02 */
} gpt_config;

typedef struct gpt_handle gpt_handle;

/* Fill *cfg with GPT-2 124M: 12 layers, 12 heads, 768 wide, MLP 3072,
 * block 1024, vocab 50257 padded to 50304, max_batch 16, bf16, AdamW
 * 0.9/0.95/1e-8, decay 0.1, clip 1.0, init std 0.02. Pure host. */
gpt_status gpt_config_default(gpt_config* cfg);

/* Bytes of device workspace a handle with this configuration needs
 * (parameters, gradients, AdamW moments, bf16 weight copies and activations
 * for max_batch x block_size tokens). Pure host; validates cfg.
 * Errors: INVALID_ARGUMENT (null, non-positive sizes, n_embd not divisible
 * by n_head, padded_vocab_size < vocab_size), UNSUPPORTED (head dim not in
 * {16, 32, 64, 128}, n_embd % 8 != 0, mlp_hidden % 8 != 0,
 * max_batch * block_size > 32768, padded_vocab_size > 131071,
 * n_embd > 2048, head_fp8 with fp32 precision or n_embd % 128 != 0). */
gpt_status gpt_workspace_bytes(const gpt_config* cfg, size_t* bytes);

/* Create a handle inside d_workspace (device memory of at least
 * gpt_workspace_bytes bytes, 256-byte aligned, owned by the caller and kept
 * alive until gpt_destroy). Parameters are initialised on `stream` from
 * `seed`: every weight is N(0, init_std) except the attention and MLP output
 * projections, N(0, init_std / sqrt(2 n_layer)) (zero with zero_init_proj);
 * biases 0, LayerNorm gains 1 ("Связанные веса и инициализация"). The normal
 * draws come from Philox4x64-10 (Salmon et al., SC'11) keyed by
 * (seed, tensor index) with counter (element / 4), turned into normals by the
 * Box-Muller transform in double precision, then rounded to fp32. AdamW
 * moments start at 0; gradients start cleared. Asynchronous.
 * Errors: INVALID_ARGUMENT, WORKSPACE_TOO_SMALL, UNSUPPORTED (as above, or
 * a device that is not gfx950), DEVICE. */
gpt_status gpt_create(const gpt_config* cfg, uint64_t seed, void* d_workspace,
                      size_t workspace_bytes, void* stream, gpt_handle** out);

/* Release host-side state. The workspace stays the caller's. */
gpt_status gpt_destroy(gpt_handle* h);

/* Run later calls on another stream (for example torch's current stream). Switching
 * to a different stream first waits for the kernel-timing events pending on the old
 * one; passing the current stream again does nothing. */
gpt_status gpt_set_stream(gpt_handle* h, void* stream);

/* One micro-step: forward pass, mean cross-entropy over the B*T positions
 * and all padded_vocab_size classes, backward pass. Gradients accumulate
 * grad_scale * d(mean loss)/d(param); the first call after gpt_create or
 * gpt_clip_and_adamw starts from zero (the training loop's zero_grad).
 * grad_scale = 1/k over k calls reproduces gradient accumulation
 * ("Накопление градиентов"). d_tokens and d_targets are device int32 [B, T]
 * read in stream order. If h_loss is non-null the call waits for the stream
 * and stores the unscaled mean loss of this micro-step.
 * Errors: INVALID_ARGUMENT (null handle or buffers, B < 1, B > max_batch,
 * T < 1, T > block_size -- the pages' "longer than block_size" failure),
 * TOKEN_RANGE (an id outside [0, padded_vocab_size); detected on the device,
 * reported by the first call that waits for the stream, which clears the
 * flag; the offending positions contribute zero, and every gpt_clip_and_adamw
 * while the flag is set leaves parameters and moments unchanged), DEVICE. */
gpt_status gpt_forward_backward(gpt_handle* h, const int32_t* d_tokens,
                                const int32_t* d_targets, int32_t B, int32_t T,
                                float grad_scale, float* h_loss);

/* Mean of the micro-step losses since the last update (the loop's
 * loss_accum). Waits for the stream. */
gpt_status gpt_loss_accum(gpt_handle* h, float* h_mean_loss);

/* Autoregressive sampling with a key/value cache ("Un GPT desde cero +
 * nanoGPT" 2.1, generate; the lecture's "Генерация и устройство", top-k
 * sampling). d_prompt: device int32 [B, T0]; d_out: device int32
 * [B, T0 + n_new], receives the prompt followed by n_new drawn tokens.
 * Each draw takes the last position's logits (after the softcap, over all
 * padded_vocab_size classes) divided by `temperature` (0 = greedy: the first
 * index of the maximum), keeps the top_k most probable tokens (0 = all; ties
 * at the k-th value go to the lower ids), and returns the first token, in id
 * order, whose cumulative kept probability exceeds u; u in (0, 1) is the top
 * 53 bits of word 0 of Philox4x64-10 at counter (draw index, row, 0, 0) with
 * key (seed, 0x73616D706C65). The prompt runs through the training forward
 * pass once (prefill); every later token runs one decode step against the
 * cached keys and values. d_logits (nullable): device fp32 [n_new, B,
 * padded_vocab_size], the logits of every draw. Uses the handle's activation
 * buffers (do not overlap with gpt_forward_backward on the same handle);
 * parameters, gradients and optimiser state are not touched. Waits for the
 * stream before returning.
 * Errors: INVALID_ARGUMENT (null buffers, B outside [1, max_batch], T0 < 1,
 * n_new < 0, T0 + n_new > block_size, temperature < 0 or not finite,
 * top_k < 0), TOKEN_RANGE (a prompt id outside [0, padded_vocab_size)),
 * DEVICE. */
gpt_status gpt_generate(gpt_handle* h, const int32_t* d_prompt, int32_t B, int32_t T0, int32_t n_new,
                        float temperature, int32_t top_k, uint64_t seed, int32_t* d_out, float* d_logits);

/* Global gradient clipping then AdamW, in two device passes:
 *   n = sqrt(sum of g^2 over every parameter, the tied wte once);
 *   c = min(1, max_grad_norm / (n + 1e-6));  g <- c g;
 *   p <- p (1 - lr weight_decay) for 2-D tensors;
 *   m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2;
 *   p <- p - lr (m / (1 - beta1^step)) / (sqrt(v / (1 - beta2^step)) + adam_eps).
 * step >= 1 is AdamW's bias-correction count. Gradients are marked for
 * clearing by the next forward_backward. If h_grad_norm is non-null the
 * call waits and returns the pre-clip norm n.
 * Errors: INVALID_ARGUMENT (step < 1, lr < 0 or not finite), NONFINITE
 * (n is not finite: parameters and moments are left unchanged; reported
 * when the call waits, i.e. with h_grad_norm non-null), TOKEN_RANGE (a
 * micro-step since the last report saw an out-of-range token or target id:
 * the update is skipped on the device; reported and cleared when the call
 * waits), DEVICE. */
gpt_status gpt_clip_and_adamw(gpt_handle* h, float lr, int32_t step, float* h_grad_norm);

/* Optimiser step with Muon on the blocks' hidden matrices (Modded-NanoGPT
 * README, technique list: "Muon optimizer"; the README gives no formula, the
 * steps are those of the article it links, K. Jordan et al., "Muon: An
 * optimizer for hidden layers in neural networks", 2024). Same clip and skip
 * rules, errors and waiting as gpt_clip_and_adamw; AdamW (learning rate lr,
 * the config's betas, eps and decay) updates the embeddings, LayerNorm gains
 * and every bias. Each h.{l}.attn.c_attn / attn.c_proj / mlp.c_fc /
 * mlp.c_proj weight W [r, c] with clipped gradient g and momentum buffer B
 * (kept where AdamW keeps its first moment; its second moment is untouched):
 *   B <- mu B + g;  u = g + mu B                       (Nesterov)
 *   X = u / (|u|_F + 1e-7), taken [c, r] when r > c;
 *   five times: A = X X^T, X <- 3.4445 X + (-4.7750 A + 2.0315 A A) X;
 *   W <- W - muon_lr sqrt(max(1, r / c)) X (oriented back), no weight decay.
 * The products and X are bf16 with fp32 accumulation on bf16 models, fp32
 * otherwise. INVALID_ARGUMENT also for muon_lr < 0 or not finite and for
 * muon_momentum outside [0, 1). */
gpt_status gpt_clip_and_muon(gpt_handle* h, float lr, float muon_lr, float muon_momentum, int32_t step,
                             float* h_grad_norm);

/* Parameter table: tensor names follow the lecture's Hugging-Face names
 * ("wte", "wpe", "h.{l}.ln_1.weight", "h.{l}.attn.c_attn.weight", ...,
 * "ln_f.bias"); linear weights are [out, in]; the tied wte appears once.
 * decay is 1 for tensors AdamW decays (every 2-D tensor). Pure host. */
gpt_status gpt_num_tensors(const gpt_handle* h, int32_t* n);
gpt_status gpt_tensor_info(const gpt_handle* h, int32_t idx, const char** name,
                           int32_t* ndim, int64_t shape[2], int32_t* decay);

/* Copy a tensor's fp32 values out of / into the model, in the canonical
 * [out, in] row-major layout. count must equal the tensor's element count;
 * buf is a device pointer if buf_on_device, else host memory. These calls
 * wait for the stream. set_param also refreshes the bf16 weight copy. */
gpt_status gpt_get_param(gpt_handle* h, int32_t idx, float* buf, int64_t count, int32_t buf_on_device);
gpt_status gpt_set_param(gpt_handle* h, int32_t idx, const float* buf, int64_t count, int32_t buf_on_device);
gpt_status gpt_get_grad(gpt_handle* h, int32_t idx, float* buf, int64_t count, int32_t buf_on_device);
gpt_status gpt_set_grad(gpt_handle* h, int32_t idx, const float* buf, int64_t count, int32_t buf_on_device);
/* AdamW first and second moments of one tensor (either pointer may be null). */
gpt_status gpt_get_opt_state(gpt_handle* h, int32_t idx, float* m, float* v, int64_t count, int32_t buf_on_device);
gpt_status gpt_set_opt_state(gpt_handle* h, int32_t idx, const float* m, const float* v, int64_t count, int32_t buf_on_device);

/* Per-position losses of the last forward_backward, fp32 [B, T] (count = B*T).
 * Waits for the stream. */
gpt_status gpt_get_row_losses(gpt_handle* h, float* buf, int64_t count, int32_t buf_on_device);

/* The lecture's learning-rate schedule ("Оптимизатор, клиппинг,
 * расписание"): max_lr (it+1)/warmup for it < warmup; min_lr for
 * it > max_steps; otherwise min_lr + 0.5 (1 + cos(pi r)) (max_lr - min_lr)
 * with r = (it - warmup)/(max_steps - warmup). Pure host. */
double gpt_lr_schedule(int32_t it, int32_t warmup_steps, int32_t max_steps, double max_lr, double min_lr);

/* Human-readable text for a status, and the last error message on a handle
 * (empty string when none). */
const char* gpt_status_string(gpt_status s);
const char* gpt_last_error(const gpt_handle* h);

/* Kernel timing (measurement support; not part of the training step).
 * gpt_set_kernel_timing takes a bit mask over kernel classes (bit c = class c,
 * -1 = all). Every launch of an enabled class, and every launch whose kernel
 * name equals the filter of gpt_set_kernel_timing_filter, is bracketed by HIP
 * events on the handle's stream. For the timed launches the library sums the
 * event time, the launch count and the algorithmic FLOPs and HBM bytes, per
 * class and per kernel name (the main kernel instantiation, as profilers name
 * it: e.g. "gemm_mfma_kernel<128, 192, 64, 2, 2, 0, 2, 2, true, true, 0, 1, 0, false>").
 * Reading the statistics synchronizes the stream. */
gpt_status gpt_set_kernel_timing(gpt_handle* h, int32_t class_mask);
gpt_status gpt_set_kernel_timing_filter(gpt_handle* h, const char* kernel_name /* null: none */);
gpt_status gpt_reset_kernel_timing(gpt_handle* h);
gpt_status gpt_num_kernel_classes(int32_t* n);
gpt_status gpt_kernel_timing(gpt_handle* h, int32_t cls, const char** name, double* total_ms,
                             int64_t* launches, double* flops, double* bytes);
/* kernel names seen in timed launches since the handle was created, in order
 * of first appearance; the returned name pointer stays valid until gpt_destroy */
gpt_status gpt_num_kernel_names(gpt_handle* h, int32_t* n);
gpt_status gpt_kernel_name_timing(gpt_handle* h, int32_t idx, const char** name, double* total_ms,
                                  int64_t* launches, double* flops, double* bytes);

#ifdef __cplusplus
}
#endif
#endif /* GPT_MI355X_H */
