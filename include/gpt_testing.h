/*
 * gpt_testing.h -- per-kernel entry points of the GPT-2 training-step library.
 *
 * Each call launches one kernel family of the training step on raw device
 * buffers, so that tests can check it against the CPU reference in isolation
 * (and, for gptk_layernorm_bwd_noalloc, so that callers that cannot allocate
 * can run the LayerNorm backward on their own buffers).
 * All pointers are device addresses owned by the caller; calls are
 * asynchronous on `stream` (a hipStream_t passed as void*) and return
 * GPT_ERR_INVALID_ARGUMENT for shapes the kernels do not accept,
 * GPT_ERR_DEVICE when the launch fails. "bf16" flags select bf16 storage for
 * the tensors documented as "act" (fp32 otherwise).
 */
#ifndef GPT_MI355X_TESTING_H
#define GPT_MI355X_TESTING_H

#include "gpt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[M, N] = epilogue(sum_k A(m,k) B(k,n)) where
 *   A(m,k) = a_kc ? A[m*lda + k] : A[k*lda + m],
 *   B(k,n) = b_kc ? B[n*ldb + k] : B[k*ldb + n]   (A, B bf16 if in_bf16 else fp32);
 * epi: 0 store (C act or fp32 by c_bf16), 1 + bias[n], 2 with y = AB + bias:
 * C = act'(y) and C2 = act(y) (act 0 = GELU tanh approximation, 1 = ReLU^2; the
 * derivative is what the backward product needs), 3 C = resid + AB + bias
 * (fp32), 4 C = AB * aux (aux act: the saved derivative), 5 C += AB (fp32). The linear-layer products of
 * the lecture's GPT ("Раздел 1 / Архитектура") in both passes reduce to these.
 * splitk_scratch (optional) holds split-K partial sums of splitk_floats floats. */
gpt_status gptk_gemm(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_kc, const void* B,
                     int64_t ldb, int32_t b_kc, void* C, int64_t ldc, int32_t in_bf16, int32_t c_bf16, int32_t epi,
                     int32_t act, const float* bias, const float* resid, const void* aux, void* C2,
                     float* splitk_scratch, int64_t splitk_floats, void* stream);

/* gptk_gemm plus the column sums of its output C (the bias gradient of a
 * layer whose output gradient C is): colsum_out[n] += sum over m of C(m, n).
 * With the ACT_GRAD epilogue on the matrix-core path without split-K the sums
 * are fused into the epilogue (fp32 values before storage rounding, per block
 * of rows, then reduced in a fixed order); otherwise a column-sum pass reads
 * the stored C. partial holds gptk_colsum_partial_floats(M, N) floats; the
 * ACCUM epilogue is not supported. */
gpt_status gptk_gemm_colsum(int32_t M, int32_t N, int32_t K, const void* A, int64_t lda, int32_t a_kc, const void* B,
                            int64_t ldb, int32_t b_kc, void* C, int64_t ldc, int32_t in_bf16, int32_t c_bf16,
                            int32_t epi, int32_t act, const float* bias, const float* resid, const void* aux, void* C2,
                            float* colsum_out, float* partial, float* splitk_scratch, int64_t splitk_floats,
                            void* stream);

/* Test control of the matrix-core GEMM: subsequent bf16 products (gptk_gemm
 * and the training step alike) use tile configuration cfg (0 <= cfg <
 * gptk_gemm_num_configs()) and split-K factor splits (0 = automatic, capped by
 * the scratch size and a minimum K slice); cfg -1 restores the automatic
 * choice. Process-wide, not thread-safe; meant for tests that cover every
 * configuration. */
gpt_status gptk_gemm_force_config(int32_t cfg, int32_t splits);
int32_t gptk_gemm_num_configs(void);

/* Test control of the matrix-core GEMM for one product shape: bf16 products
 * with these M, N, K and operand layouts (gptk_gemm and the training step
 * alike) use tile configuration cfg with `splits` k-slices (splits 0 = 1);
 * cfg -1 drops the override. A gptk_gemm_force_config setting takes
 * precedence. Process-wide, not thread-safe; meant for measurements that
 * compare configurations of single products inside the whole step. */
gpt_status gptk_gemm_tune(int32_t M, int32_t N, int32_t K, int32_t a_kc, int32_t b_kc, int32_t cfg, int32_t splits);

/* The FP8 head's product (Modded-NanoGPT README technique list, FP8 matmul for
 * the output head): C [M, N] bf16 = (e4m3(A s_a) . e4m3(B s_b)^T) / (s_a s_b)
 * for bf16 A [M, K] and B [N, K] (row-major, k-contiguous), s = 448 / max|t|
 * per tensor in fp32, e4m3 rounding to nearest even. K % 128 == 0, N % 8 == 0,
 * 16-byte aligned buffers; scratch (256-byte aligned) holds
 * gptk_gemm_fp8_scratch_bytes(M, N, K) bytes: the e4m3 copies, the scales
 * (floats 0..3: 1/s_a, 1/s_b, s_a, s_b) and the max-reduction partials. */
gpt_status gptk_gemm_fp8(int32_t M, int32_t N, int32_t K, const void* A, const void* B, void* C, void* scratch,
                         int64_t scratch_bytes, void* stream);
int64_t gptk_gemm_fp8_scratch_bytes(int32_t M, int32_t N, int32_t K);

/* Muon's orthogonalisation of one matrix (the iteration of gpt_clip_and_muon
 * on a single gradient, momentum 0): O [r, c] (fp32, row-major) = the five
 * quintic Newton-Schulz steps applied to G [r, c] (fp32, row-major) normalised
 * by |G|_F + 1e-7, iterates and products bf16 with fp32 accumulation when
 * bf16, fp32 otherwise. scratch (256-byte aligned) holds
 * gptk_muon_scratch_bytes(r, c, bf16) bytes. */
gpt_status gptk_muon_orthogonalize(int32_t r, int32_t c, const float* G, float* O, int32_t bf16, void* scratch,
                                   int64_t scratch_bytes, void* stream);
int64_t gptk_muon_scratch_bytes(int32_t r, int32_t c, int32_t bf16);

/* Causal (optionally windowed: i - j < window) softmax(Q K^T / sqrt(hd)) V per
 * (batch, head), heads interleaved in the columns of row-major [B*T, *]
 * buffers ("El Mecanismo de Atención"). Forward writes o and lse [B, H, T];
 * backward also computes D = rowsum(dO o O) into D [B, H, T] and writes dq,
 * dk, dv (row stride ldd). */
gpt_status gptk_attention(int32_t backward, int32_t B, int32_t T, int32_t H, int32_t hd, int32_t window,
                          const void* q, const void* k, const void* v, int64_t ldq, int64_t ldk, int64_t ldv,
                          void* o, int64_t ldo, float* lse, const void* dO, int64_t lddo, float* D, void* dq, void* dk,
                          void* dv, int64_t ldd, int32_t bf16, void* stream);

/* Attention backward into one [B*T, 3*H*hd] buffer dqkv (dq, dk, dv column
 * blocks, row stride 3*H*hd) plus the qkv bias gradient: colsum_out[c] += sum
 * over rows of dqkv[:, c]. On the matrix-core path the sums are fused into the
 * backward kernels (fp32 values before storage rounding, per 128-row block of a
 * sequence, reduced in a fixed order); otherwise a column-sum pass reads dqkv.
 * partial holds gptk_attention_colsum_partial_floats(B, T, H, hd) floats; the
 * other arguments are those of gptk_attention's backward. */
gpt_status gptk_attention_bwd_colsum(int32_t B, int32_t T, int32_t H, int32_t hd, int32_t window, const void* q,
                                     const void* k, const void* v, int64_t ldq, int64_t ldk, int64_t ldv, const void* o,
                                     int64_t ldo, const float* lse, const void* dO, int64_t lddo, float* D, void* dqkv,
                                     int32_t bf16, float* colsum_out, float* partial, void* stream);
int64_t gptk_attention_colsum_partial_floats(int32_t B, int32_t T, int32_t H, int32_t hd);

/* LayerNorm over rows of width d with biased variance. Forward: y (act),
 * mean, rstd. Backward: dres = (overwrite ? 0 : dres) + dx, optional bf16
 * copy dres_lp, dg += sum dy xhat, db += sum dy, and (dcol nullable) dcol +=
 * column sums of the resulting dres; partial holds
 * gptk_layernorm_partial_floats(M, d) floats. */
gpt_status gptk_layernorm(int32_t backward, int32_t M, int32_t d, float eps, const float* x, const float* g,
                          const float* b, void* y, float* mean, float* rstd, const float* dy, float* dres,
                          void* dres_lp, int32_t overwrite, float* dg, float* db, float* dcol, float* partial,
                          int32_t bf16, void* stream);
int64_t gptk_layernorm_partial_floats(int32_t M, int32_t d);

/* The LayerNorm backward of gptk_layernorm (backward = 1) for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): same arguments without `partial`,
 * same kernels and results. The partial sums live in a device array inside
 * the library, one per GPU, of gptk_layernorm_noalloc_max_floats() floats
 * (32 MiB, held until the process ends); the call allocates nothing.
 * A shape whose gptk_layernorm_partial_floats(M, d) exceeds that size is
 * rejected with GPT_ERR_INVALID_ARGUMENT (every shape with M <= 32768 and
 * d <= 2048 fits). Calls that overlap on one GPU share the array and race;
 * calls in stream order do not. dg and db are required, dcol and dres_lp
 * nullable. GPT_ERR_DEVICE if the array's address cannot be obtained. */
gpt_status gptk_layernorm_bwd_noalloc(int32_t M, int32_t d, const float* x, const float* g, const float* mean,
                                      const float* rstd, const float* dy, float* dres, void* dres_lp,
                                      int32_t overwrite, float* dg, float* db, float* dcol, int32_t bf16,
                                      void* stream);
int64_t gptk_layernorm_noalloc_max_floats(void);

/* Fused softmax cross-entropy on logits z [M, Vp] (act, overwritten in place
 * by the gradient (softmax - onehot) * gscale); optional tanh softcap. */
gpt_status gptk_cross_entropy(int32_t M, int32_t Vp, void* z, const int32_t* y, float* row_loss, float gscale,
                              float cap, int32_t* err, int32_t bf16, void* stream);

/* The speedrun block's query/key preparation (Modded-NanoGPT README (oa0.com),
 * technique list: QK-Norm then rotary positions): per row m (position m % T),
 * head h and each of q and k, parameter-free RMS normalisation over the head's
 * hd values (norm = 1; eps inside the root) and the rotary rotation of each
 * rotate-half pair (i, i + hd/2) by the angle (m % T) * base^(-2i/hd)
 * (rope = 1). backward = 0: qkv [M, 3 H hd] (q = columns [0, H hd), k the next
 * H hd) -> out [M, 2 H hd] (q then k). backward = 1: out is dqkv [M, 3 H hd],
 * whose q and k parts (gradients at the prepared q and k) are replaced in
 * place by the gradients at the raw q and k, given the same qkv. tables:
 * caller-owned device scratch of T * hd floats (the cos and sin tables,
 * rebuilt on every call). bf16 selects bf16 storage of qkv and out. hd even,
 * at most 128; anything else is GPT_ERR_INVALID_ARGUMENT. */
gpt_status gptk_qk_prep(int32_t backward, int32_t M, int32_t T, int32_t H, int32_t hd, const void* qkv, void* out,
                        float* tables, double base, int32_t norm, int32_t rope, float eps, int32_t bf16,
                        void* stream);

/* dwte[tok[m]] += dx[m] and dwpe[t] += sum_b dx[b, t] (dwpe may be null),
 * deterministic and atomic-free; scratch holds gptk_embed_bwd_scratch_bytes. */
gpt_status gptk_embed_bwd(const int32_t* tok, const float* dx, float* dwte, float* dwpe, int32_t B, int32_t T,
                          int32_t d, int32_t Vp, void* scratch, void* stream);
int64_t gptk_embed_bwd_scratch_bytes(int32_t M, int32_t d);

/* One draw per row of fp32 logits [B, Vp] into tokens[b], by the sampler of
 * gpt_generate (the logit softcap applied in place first when cap > 0):
 * temperature 0 takes the first index of the largest logit; otherwise the
 * weights exp((z - max) / temperature), restricted for 0 < top_k < Vp to the
 * top_k largest logits (lower indices first among equal values), and the
 * token is the first in token order whose running weight exceeds u times
 * their sum, u = ((x >> 11) + 0.5) 2^-53 for the first output word x of
 * Philox4x64-10 at counter (step, b, 0, 0) with key (seed, sampling stream);
 * "Un GPT desde cero + nanoGPT" 2.1, generate, and the lecture's "Генерация
 * и устройство", top-k 50. Device pointers; logits is modified when
 * cap > 0. Invalid sizes return GPT_ERR_INVALID_ARGUMENT. */
gpt_status gptk_sample(float* logits, int32_t B, int32_t Vp, float cap, float temperature, int32_t top_k, uint64_t seed,
                       int32_t step, int32_t* tokens, void* stream);

/* out[n] += sum_m Y[m*ld + n] (bias gradients); partial holds
 * gptk_colsum_partial_floats(M, N) floats. */
gpt_status gptk_colsum(int32_t M, int32_t N, const void* Y, int64_t ld, int32_t bf16, float* out, float* partial,
                       void* stream);
int64_t gptk_colsum_partial_floats(int32_t M, int32_t N);

#ifdef __cplusplus
}
#endif
#endif /* GPT_MI355X_TESTING_H */
