// Host-side launch functions for the gfx950 kernels of the GPT-2 training
// step. All launches are asynchronous on the given stream; every pointer is a
// device address. `bf` selects bf16 (true) or fp32 (false) storage of the
// activation tensors named "act" below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gk {

// ---------------------------------------------------------------- init / fills
// dst[e] = fp32(std * z_e), z from Philox4x64-10 keyed (seed, stream_id),
// counter e/4, Box-Muller pairs (words 0,1) and (2,3) in double precision.
void init_normal(float* dst, int64_t n, uint64_t seed, uint64_t stream_id, double std, hipStream_t s);
void fill_f32(float* dst, int64_t n, float value, hipStream_t s);
void fill_i32(int32_t* dst, int64_t n, int32_t value, hipStream_t s);
void f32_to_bf16(void* dst, const float* src, int64_t n, hipStream_t s);
// rotary tables cos/sin [T, hd/2] of the angle t * base^(-2i/hd) (double precision math)
void rope_tables(float* cos_t, float* sin_t, int T, int hd, double base, hipStream_t s);

// ---------------------------------------------------------------- embedding
// x0[m, :] = wte[tok[m], :] (+ wpe[m % T, :] if wpe); fp32 out. Invalid ids
// give a zero token row and set *err = 1.
void embed_fwd(const int32_t* tok, const float* wte, const float* wpe, float* x0, int M, int T, int d,
               int Vp, int32_t* err, hipStream_t s);

// Deterministic, atomic-free dwte[tok[m]] += dx[m] and dwpe[t] += sum_b dx[b, t].
// scratch needs embed_bwd_scratch_bytes(M, d) bytes.
size_t embed_bwd_scratch_bytes(int M, int d);
void embed_bwd(const int32_t* tok, const float* dx, float* dwte, float* dwpe, int B, int T, int d, int Vp,
               void* scratch, hipStream_t s);
// embed_bwd in two parts: the token sort (depends on the tokens only, so it
// can run early on another stream) and the accumulation that reads dx.
void embed_bwd_sort(const int32_t* tok, int B, int T, int d, int Vp, void* scratch, hipStream_t s);
// dwte rows += their dx rows; dwpe (+)= the position sums (overwritten when
// overwrite_wpe: the first contribution of a pass whose gradients start empty).
void embed_bwd_accumulate(const float* dx, float* dwte, float* dwpe, int B, int T, int d, void* scratch,
                          hipStream_t s, bool overwrite_wpe = false);

// ---------------------------------------------------------------- LayerNorm
// y = (x - mean) rstd * g + b over rows of width d (fp32 x, act y); saves mean, rstd.
void layernorm_fwd(bool bf, const float* x, const float* g, const float* b, void* y, float* mean,
                   float* rstd, int M, int d, float eps, hipStream_t s);
// dres (+)= LN backward of dy; writes a bf16 copy of dres when dres_lp != null;
// dg += sum dy*xhat, db += sum dy, and (if dcol) dcol += column sums of the
// resulting dres (deterministic two-pass); partial needs
// layernorm_bwd_partial_floats(M, d) floats.
size_t layernorm_bwd_partial_floats(int M, int d);
void layernorm_bwd(bool bf, const float* dy, const float* x, const float* mean, const float* rstd,
                   const float* g, float* dres, void* dres_lp, bool overwrite, float* dg, float* db,
                   float* dcol, float* partial, int M, int d, hipStream_t s);

// layernorm_bwd with its partial sums in a file-scope device array of
// layernorm_bwd_static_capacity_floats() floats instead of a caller buffer
// (nothing allocated). Returns 0, -1 when the shape needs more than the
// array holds, -4 on a HIP runtime failure.
size_t layernorm_bwd_static_capacity_floats();
int layernorm_bwd_static(bool bf, const float* dy, const float* x, const float* mean, const float* rstd,
                         const float* g, float* dres, void* dres_lp, bool overwrite, float* dg, float* db,
                         float* dcol, int M, int d, hipStream_t s);

// ---------------------------------------------------------------- column sums
// out[n] += sum_m Y[m, n] (Y act or fp32 with row stride ld); partial needs
// colsum_partial_floats(M, N) floats.
size_t colsum_partial_floats(int M, int N);
void colsum(bool y_bf, const void* Y, int64_t ld, int M, int N, float* out, float* partial, hipStream_t s);

// Forms that only launch the row pass and leave the partial sums for
// reduce_jobs: layernorm_bwd_rows writes [3][nb][d] (dgamma, dbeta, column
// sums of the new dres; nb = layernorm_bwd_num_partials(M)), colsum_rows
// writes [np][N] (np = colsum_num_partials(M)).
int layernorm_bwd_num_partials(int M);
void layernorm_bwd_rows(bool bf, const void* dy, bool dy_bf, const float* x, const float* mean, const float* rstd,
                        const float* g, float* dres, void* dres_lp, bool overwrite, float* partial, int M, int d,
                        hipStream_t s);   // dy bf16 when dy_bf (bf16 path only), else fp32
int colsum_num_partials(int M);
void colsum_rows(bool y_bf, const void* Y, int64_t ld, int M, int N, float* partial, hipStream_t s);

// Deferred column reductions: for each job, out[c] += sum over p < np of
// part[p * n + c], c < n, summed in a fixed order (groups of 64 partial rows,
// then the groups in order), all jobs in two launches. jobs is a device array;
// tmp holds reduce_jobs_tmp_floats(njobs, max_np, max_n) floats, max_np and
// max_n bounding every job's np and n.
struct RedJob {
    const float* part;
    float* out;
    int np, n;
};
size_t reduce_jobs_tmp_floats(int njobs, int max_np, int max_n);
// out[c] += sum over p < np of part[p * n + c] (one job, the same fixed order);
// tmp holds ceil(np / 64) * n floats
void reduce_rows(const float* part, int np, int n, float* out, float* tmp, hipStream_t s);
// every job's out (+)= its partial sums; overwrite stores them instead (the
// first contribution to outputs that no earlier work of the pass wrote)
void reduce_jobs(const RedJob* jobs, int njobs, int max_np, int max_n, float* tmp, hipStream_t s,
                 bool overwrite = false);

// ---------------------------------------------------------------- cross-entropy
// Per row of logits z (act, [M, Vp], in place): z' = cap tanh(z/cap) if cap > 0;
// loss_m = logsumexp(z') - z'[y_m]; z <- (softmax(z') - onehot(y)) * gscale
// (times 1 - tanh^2 with the cap). Invalid targets: loss 0, zero row, *err = 1.
void cross_entropy(bool bf, void* z, const int32_t* y, float* row_loss, int M, int Vp, float gscale,
                   float cap, int32_t* err, hipStream_t s);
// *loss_out = mean(row_loss[0..M)); *loss_sum += that mean (deterministic),
// or = that mean when first.
void mean_loss(const float* row_loss, int M, float* loss_out, float* loss_sum, hipStream_t s, bool first = false);

// ---------------------------------------------------------------- attention helpers
// D[b, h, t] = sum_c dO[m, h*hd + c] * O[m, h*hd + c]
void attn_rowdot(bool bf, const void* dO, const void* O, float* D, int B, int T, int H, int hd, hipStream_t s);
// q/k RMS normalisation (no gain) then rotary rotation, per head.
// fwd: reads q,k from qkv [M, 3d], writes qk_out [M, 2d]; row m is at
// position pos0 + m % T.
void qk_prep_fwd(bool bf, const void* qkv, void* qk_out, const float* cos_t, const float* sin_t, int M, int T,
                 int H, int hd, int norm, int rope, float eps, hipStream_t s, int pos0 = 0);
// bwd: in place on the q,k columns of dqkv [M, 3d], raw q,k re-read from qkv.
void qk_prep_bwd(bool bf, const void* qkv, void* dqkv, const float* cos_t, const float* sin_t, int M, int T,
                 int H, int hd, int norm, int rope, float eps, hipStream_t s);

// ---------------------------------------------------------------- sampling with a key/value cache
// x[b] = wte[seq[b * ld + pos]] + wpe[pos] (wpe nullable); invalid ids set *err.
void gen_embed(const int32_t* seq, int64_t ld, int pos, const float* wte, const float* wpe, float* x, int B, int d,
               int Vp, int32_t* err, hipStream_t s);
// cache rows: dst[(b Tmax + t0 + t) d + c] = src[(b nt + t) src_ld + c] (act), d % 8 == 0
void cache_put(bool bf, const void* src, int64_t src_ld, void* dst, int B, int nt, int Tmax, int t0, int d,
               hipStream_t s);
// out [B, d] (act): per (b, head) softmax(q k^T / sqrt(hd)) v over cached keys
// j0 .. pos (j0 = pos - window + 1 with a window, else 0); caches [B, Tmax, d].
// The key and value of position pos (rows b of knew and vnew, strides ldk and
// ldv) are first written into the caches by the same workgroups.
void gen_attention(bool bf, const void* q, int64_t ldq, const void* knew, int64_t ldk, const void* vnew, int64_t ldv,
                   void* kc, void* vc, void* out, int B, int H, int hd, int pos, int Tmax, int window, hipStream_t s);
// One draw per row of fp32 logits [B, Vp] (softcapped in place when cap > 0,
// copied to logits_out when non-null) into seq[b * ld_seq + pos_out].
void gen_sample(float* logits, int B, int Vp, float cap, float temperature, int top_k, uint64_t seed, int step,
                int32_t* seq, int64_t ld_seq, int pos_out, float* logits_out, hipStream_t s);

// ---------------------------------------------------------------- optimiser
// norm = sqrt(sum g^2); coef = min(1, max_norm / (norm + 1e-6)); *skip = 1 when
// the norm is not finite or *id_err (nullable) is set, else 0.
// partial needs 1024 doubles.
void grad_norm(const float* g, int64_t n, double* partial, float* norm_out, float* coef_out,
               int32_t* skip, const int32_t* id_err, float max_norm, hipStream_t s);
// AdamW over the flat buffers; elements [0, n_decay) are decayed and mirrored
// to the bf16 copy wbf (if non-null). Skips everything when *skip.
void adamw(float* p, const float* g, float* m, float* v, void* wbf, int64_t n, int64_t n_decay,
           const float* coef, const int32_t* nonfinite, float lr, float b1, float b2, float eps, float wd,
           float rbc1, float rbc2, hipStream_t s);

// ---------------------------------------------------------------- GEMM
enum GemmEpi {
    EPI_STORE = 0,      // C = A B                        (C: act or fp32)
    EPI_BIAS = 1,       // C = A B + bias                 (C: act)
    EPI_BIAS_ACT = 2,   // y = A B + bias; C = act'(y); C2 = act(y)   (C, C2: act)
    EPI_BIAS_RESID = 3, // C = resid + A B + bias         (C, resid: fp32)
    EPI_ACT_GRAD = 4,   // C = (A B) * aux, aux = act' saved by EPI_BIAS_ACT   (C, aux: act)
    EPI_ACCUM = 5       // C += A B                       (C: fp32)
};
struct Gemm {
    int M, N, K;
    const void* A; int64_t lda; bool a_kc;   // A(m,k) = a_kc ? A[m*lda + k] : A[k*lda + m]
    const void* B; int64_t ldb; bool b_kc;   // B(k,n) = b_kc ? B[n*ldb + k] : B[k*ldb + n]
    void* C; int64_t ldc; bool c_bf;         // output storage type
    void* C2;
    const float* bias;
    const float* resid;
    const void* aux;
    int epi;
    int act;
    bool in_bf;                              // A and B storage (bf16 or fp32)
    // e4m3 products only: the bf16 store is multiplied by out_scale[0] * out_scale[1]
    const float* out_scale = nullptr;
    // decode-shaped products only (skinny_gemm): when ln_g is set, A is the
    // fp32 residual stream and the product takes LayerNorm(A; ln_g, ln_b, ln_eps)
    // rounded to bf16, as the separate LayerNorm kernel would store it
    const float* ln_g = nullptr;
    const float* ln_b = nullptr;
    float ln_eps = 0.f;
    // ACT_GRAD epilogue, plans with bm > 0: cpart[(m / bm) * N + n] = sum over
    // the rows m of one bm-row block of the fp32 output values (column sums
    // for a bias gradient, reduced later)
    float* cpart = nullptr;
    // batched products (STORE epilogue only, no split-K): entry b reads A + b sa
    // and B + b sb and writes C + b sc (element strides)
    int batch = 1;
    int64_t sa = 0, sb = 0, sc = 0;
};
// How a product runs: kernel (matrix-core tile configuration, or cfg = -1
// for the portable kernel), split-K factor, and the name of the main kernel
// instantiation (as profilers print it).
struct GemmPlan {
    int cfg = -1;
    int splits = 1;
    int bm = 0;      // rows per block of fused column sums (0: the plan cannot produce them)
    char name[112] = {0};
};
// scratch: split-K partials for the matrix-core kernel (may be null: no split)
GemmPlan gemm_plan(const Gemm& g, size_t splitk_floats);
// main kernel, then (split-K only) the kernel that sums the slices
void gemm_main(const Gemm& g, const GemmPlan& p, float* splitk_scratch, hipStream_t s);
void gemm_finish(const Gemm& g, const GemmPlan& p, const float* splitk_scratch, hipStream_t s);
void gemm(const Gemm& g, float* splitk_scratch, size_t splitk_floats, hipStream_t s);
// Products of a decode step: bf16 (or, with ln_g, a LayerNorm of fp32 rows) A
// and bf16 W, both k-contiguous, M <= 16, K % 32 == 0, K <= 4096, epilogues
// STORE / BIAS / BIAS_ACT / BIAS_RESID.
bool skinny_gemm_ok(const Gemm& g);
void skinny_gemm(const Gemm& g, hipStream_t s);
// e4m3 product for the FP8 head: C [M, N] bf16 (row stride ldc) =
// (A8 [M, K] . B8 [N, K]^T) * inv_sa * inv_sb, A8 and B8 e4m3 bytes with row
// strides lda and ldb (bytes), K % 128 == 0, lda % 16 == ldb % 16 == 0.
void gemm_f8(int M, int N, int K, const void* A8, int64_t lda, const void* B8, int64_t ldb, void* C, int64_t ldc,
             const float* inv_sa_sb, hipStream_t s);
// Muon for the hidden matrices (muon.hip), a batch of same-shaped W_e [r, c]
// at element stride os in the flat parameter, gradient and buffer arrays.
// muon_direction: buf <- mu buf + coef g, u_e = coef g + mu buf written wide
// ([c, r] when r > c) at u + e r c, scale[e] = 1 / (|u_e|_F + 1e-7) (part: ps >=
// muon_part_floats(r, c) floats per entry). muon_newton_schulz: five quintic
// iterations on X_e [m, n] = u_e * scale[e] (m <= n; X0, X1 batch m n and A, AA,
// Bp batch m m elements, bf16 when bf), returning the buffer with the results.
// muon_apply: W_e -= step * X_e oriented back, bf16 shadow wbf (nullable, same
// stride) refreshed. The momentum and apply kernels do nothing when *nonfinite
// is set.
int64_t muon_part_floats(int r, int c);
void muon_direction(const float* g, float* buf, int64_t os, int batch, float* u, float* part, int64_t ps, int r, int c,
                    float mu, const float* coef, const int32_t* nonfinite, float* scale, hipStream_t s);
void* muon_newton_schulz(bool bf, const float* u, const float* scale, int m, int n, int batch, void* X0, void* X1,
                         void* A, void* AA, void* Bp, float* splitk, size_t splitk_floats, hipStream_t s);
void muon_apply(bool bf, float* W, void* wbf, int64_t os, int batch, const void* X, int r, int c, float step,
                const int32_t* nonfinite, hipStream_t s);
// Per-tensor e4m3 quantisation of a bf16 tensor (n % 8 == 0):
// *scale = 448 / max|x| (1 for an all-zero tensor), *inv = 1 / *scale,
// q = e4m3(fp32(x) * scale) rounded to nearest even (saturating at 448);
// part holds 1024 floats.
void quantize_e4m3(const void* x, int64_t n, uint8_t* q, float* scale, float* inv, float* part, hipStream_t s);
// test control of the matrix-core tile configuration / split-K (cfg -1: automatic)
void gemm_mfma_force(int cfg, int splits);
int gemm_mfma_num_configs();
// test control: the product of shape (M, N, K, a_kc, b_kc) uses tile
// configuration cfg with `splits` k-slices (cfg -1 drops the override); 0 or -1 on a bad argument
int gemm_mfma_tune(int M, int N, int K, bool a_kc, bool b_kc, int cfg, int splits);

// ---------------------------------------------------------------- attention
struct Attn {
    int B, T, H, hd, window;
    const void* q; const void* k; const void* v; int64_t ldq, ldk, ldv;   // row strides
    void* o; int64_t ldo;
    float* lse;                       // [B, H, T]
    const void* dO; int64_t lddo;     // backward
    const float* D;                   // [B, H, T]: rowsum(dO o O), read by the backward kernels
    float* Dout;                      // where the matrix-core backward computes it (same buffer)
    void* dq; void* dk; void* dv; int64_t ldd;
    bool bf;
    // backward, matrix-core path: when set, the fp32 column sums (values before
    // rounding) of dq, dk, dv over each 128-row block of a sequence, row
    // b * ceil(T / 128) + block, columns [dq heads | dk heads | dv heads] (3 H hd)
    float* cpart = nullptr;
};
void attention_fwd(const Attn& a, hipStream_t s);
// backward: computes D itself (into Dout) when the matrix-core kernels run;
// the portable kernels need D precomputed (attn_rowdot)
// returns true when the matrix-core kernels ran (and wrote a.cpart if set)
bool attention_bwd(const Attn& a, hipStream_t s);

}  // namespace gk
