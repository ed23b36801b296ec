/*
 * tt.h — C ABI of libtt, an MI355X (gfx950) GPT-2 training step.
 *
 * Sources (page titles abbreviated):
 *   tinytorch page  "不用PyTorch，一个头文件就能训练GPT-2：Arena内存池+自动微分的C++实现"
 *   Forge page      "17岁少年用C++从零构建深度学习框架Forge，精确复现GPT-2"
 *   C++/CUDA page   "从零手写C++深度学习框架：Tensor设计、Autograd与CUDA优化实战"
 *   define-by-run   "为什么我要从零写一个深度学习框架" (NumPy autograd tutorial)
 *   microcrad page  "microcrad" (micrograd in C)
 *
 * General conventions
 *   - Every pointer argument is a DEVICE pointer unless marked [host].
 *   - All arrays are dense row-major.  A linear layer is y = x·W + b with W of
 *     shape [in, out] (tinytorch page, §3 item 3: C[M,N] = A[M,K]·B[K,N]).
 *   - Every call only validates arguments on the host and enqueues kernels on
 *     the context's HIP stream; it returns before the GPU work finishes.
 *     Nothing aborts: every call returns a tt_status (0 on success, negative
 *     on failure — the convention of microcrad's value_backward).  On a
 *     validation failure nothing is enqueued.  Asynchronous device faults and
 *     in-kernel range errors (a token id or target outside [0, V)) surface at
 *     tt_ctx_sync().
 *   - Gradient outputs marked "+=" ACCUMULATE into what the caller passes, the
 *     rule the tinytorch page states for tensors with several consumers
 *     (§3 item 3) and the define-by-run page illustrates with 2 + 3 = 5
 *     (§3.2).  The caller zeroes them (microcrad "反向传播" section;
 *     tinytorch §3 item 7, ZeroGrad before Backward).  tt_train_step zeroes
 *     its own gradient buffer.
 *   - Precision modes.  TT_F32: every tensor float32 and float32 arithmetic.
 *     TT_BF16: GEMM and attention operands bf16 with float32 accumulation;
 *     master weights, gradients, optimizer moments, the residual stream,
 *     LayerNorm statistics and the loss stay float32 (C++/CUDA page §3.4:
 *     fp32 master weights with low-precision compute).  A "mode tensor" below
 *     is float32 in TT_F32 and bf16 (uint16 storage, round to nearest even)
 *     in TT_BF16.  TT_FP16: as TT_BF16 with IEEE binary16 in place of bf16
 *     (the same page's FP16 variant); the whole-model step then scales its
 *     loss gradient dynamically (tt_model_loss_scale_*).
 *   - Alignment: device pointers must be 16-byte aligned; row lengths need not
 *     be tile multiples (ragged edges are handled).
 *   - One context per stream; a context is not thread-safe.
 */
#ifndef TT_H
#define TT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TT_OK = 0,
  TT_EINVAL = -1,       /* bad argument: NULL, shape, alignment, mode           */
  TT_ENOMEM = -2,       /* arena exhausted, or device allocation failed          */
  TT_EHIP = -3,         /* HIP runtime error (text in tt_ctx_last_error)         */
  TT_ESTALE = -4,       /* handle whose magic word does not match (freed/foreign)*/
  TT_ENONFINITE = -5,   /* a non-finite value was detected                       */
  TT_EUNSUPPORTED = -6, /* shape outside what the kernels support (e.g. hs!=64)  */
  TT_ERANGE = -7        /* a token id or target was outside [0, V) (device check)*/
} tt_status;

typedef enum { TT_F32 = 0, TT_BF16 = 1, TT_FP16 = 2 } tt_mode;

typedef struct tt_ctx tt_ctx;
typedef struct tt_model tt_model;

/* ------------------------------------------------------------------------ */
/* Context and HBM arena.                                                    */
/* The tinytorch page (§3 item 1) carves every tensor out of one pre-allocated */
/* block by bumping an offset and frees all intermediates at once by resetting */
/* it.  Here the block lives in HBM: one hipMalloc (or caller-owned memory),   */
/* bumped with 256-byte alignment; tt_ctx_mark() fixes what stays and          */
/* tt_ctx_reset() returns the offset to the mark.                             */
/* ------------------------------------------------------------------------ */

/* device: HIP device ordinal.  hip_stream: hipStream_t to enqueue on (NULL =
 * the null stream).  arena_bytes: arena size.  arena_base: nullable; when
 * given, caller-owned device memory of arena_bytes bytes (e.g. a torch
 * buffer) that must outlive the context; when NULL the context hipMallocs the
 * arena and frees it in tt_ctx_destroy.  *out [host] receives the handle.
 * Errors: TT_EINVAL, TT_ENOMEM, TT_EHIP. */
int tt_ctx_create(int device, void *hip_stream, size_t arena_bytes, void *arena_base,
                  tt_ctx **out);
/* NULL-safe (microcrad: releasing NULL is a no-op).  Frees only what the
 * context allocated.  Waits for the stream first. */
void tt_ctx_destroy(tt_ctx *ctx);
/* Change the stream later calls enqueue on. */
int tt_ctx_set_stream(tt_ctx *ctx, void *hip_stream);
/* Bump-allocate bytes (align: power of two, at least 256 is used).  *dptr
 * [host] receives a device pointer valid until the next tt_ctx_reset() below
 * it or tt_ctx_destroy().  TT_ENOMEM when the arena is exhausted. */
int tt_ctx_alloc(tt_ctx *ctx, size_t bytes, size_t align, void **dptr);
/* Make everything allocated so far persistent. */
int tt_ctx_mark(tt_ctx *ctx);
/* Return the offset to the last mark (tinytorch §3 item 1, Reset()). */
int tt_ctx_reset(tt_ctx *ctx);
/* Bytes in use / capacity ([host] outputs, either may be NULL). */
int tt_ctx_usage(const tt_ctx *ctx, size_t *used, size_t *capacity);
/* Wait for the stream; report asynchronous HIP errors (TT_EHIP) and in-kernel
 * range errors (TT_ERANGE, then cleared). */
int tt_ctx_sync(tt_ctx *ctx);
const char *tt_strerror(int status);
const char *tt_ctx_last_error(const tt_ctx *ctx);

/* Kernel timing (the C++/CUDA page, section 2.2, records an event pair per
 * op on its stream).  tt_ctx_profile(ctx, 1) clears earlier records and
 * starts bracketing every kernel launch with HIP events on the context's
 * stream; tt_ctx_profile(ctx, 0) stops.  tt_ctx_profile_report waits for the
 * stream and aggregates the records by kernel name: calls, total
 * milliseconds, and the algorithmic work of those launches (FLOPs for
 * matrix-core kernels, HBM bytes for bandwidth-bound ones; 0 where the other
 * measure applies).  out [host] may be NULL to query *count; otherwise it
 * holds *count entries on input and *count receives the number of kernels.
 * Names point to static strings inside the library. */
typedef struct {
  const char *name;
  int calls;
  double ms;
  double flops;
  double bytes;
} tt_prof_entry;
int tt_ctx_profile(tt_ctx *ctx, int enable);
int tt_ctx_profile_report(tt_ctx *ctx, tt_prof_entry *out /* [host] */, int *count /* [host] */);

/* ------------------------------------------------------------------------ */
/* Op level.                                                                 */
/* ------------------------------------------------------------------------ */

typedef enum {
  TT_EPI_NONE = 0,     /* Y = X·W + b                                   (Y mode)   */
  TT_EPI_GELU = 1,     /* P = X·W + b stored in preact; Y = GELU_tanh(P)  (mode)    */
  TT_EPI_RESIDUAL = 2  /* Y = resid + X·W + b                           (Y float32)*/
} tt_epilogue;

/* Linear forward — tinytorch page §3 item 3 (MatMulForward), §3 item 4 (GELU,
 * tanh form), §4 (residual connection x + f(x)).
 * X [M,K] mode tensor, W [K,N] mode tensor, b [N] float32 (nullable).
 * Y [M,N]: mode tensor for NONE/GELU, float32 for RESIDUAL.  resid [M,N]
 * float32 (RESIDUAL only; may equal Y).  preact [M,N] mode tensor (GELU only,
 * nullable: then not stored).  M, K, N >= 1. */
int tt_linear_fwd(tt_ctx *ctx, tt_mode mode, int M, int K, int N, const void *X,
                  const void *W, const float *b, void *Y, int epilogue, const float *resid,
                  void *preact);

/* Linear backward — tinytorch page §3 item 3 (MatMulBackward: dA += dC·Bᵀ,
 * dB += Aᵀ·dC); define-by-run page §3.2 (same shapes).
 * X [M,K], W [K,N], dY [M,N]: mode tensors.  dX [M,K] float32, nullable:
 * written (accumulate_dX = 0) or += (accumulate_dX != 0).  dW [K,N] float32
 * +=, nullable.  db [N] float32 +=, nullable (column sums of dY). */
int tt_linear_bwd(tt_ctx *ctx, tt_mode mode, int M, int K, int N, const void *X,
                  const void *W, const void *dY, float *dX, float *dW, float *db,
                  int accumulate_dX);

/* LayerNorm forward — tinytorch page §4 (subtract the mean, divide by the
 * standard deviation, scale, shift); Forge page "最硬的一关" (epsilon placement
 * and variance method matter).  Biased variance, eps inside the square root:
 *   y = (x - mean) * rstd * g + b,  rstd = 1/sqrt(mean((x-mean)^2) + eps).
 * x [N,C] float32; g, b [C] float32; y [N,C] mode tensor; mean, rstd [N]
 * float32 (nullable).  1 <= C <= 4096, C % 4 == 0. */
int tt_layernorm_fwd(tt_ctx *ctx, tt_mode mode, int N, int C, float eps, const float *x,
                     const float *g, const float *b, void *y, float *mean, float *rstd);

/* LayerNorm backward (chain rule of the above).  dy [N,C] float32.
 * dx [N,C] float32 +=.  dg, db [C] float32 +=.  Same C limits.  The column
 * sums behind dg and db are formed per workgroup into a partial-sum
 * workspace (arena scratch) and then added up by a second launch. */
int tt_layernorm_bwd(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                     const float *mean, const float *rstd, const float *g, const float *dy,
                     float *dx, float *dg, float *db);
/* Size in bytes of that workspace for every N <= n_rows rows of width C
 * (host only, no GPU needed): the number of workgroups does not grow
 * monotonically with N (each wave takes 2, 4 or 8 rows depending on N), so
 * this is the maximum over N.  TT_EINVAL for a C the kernels do not take. */
int tt_layernorm_bwd_workspace(int n_rows, int C, size_t *bytes);
/* tt_layernorm_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, layout and results as tt_layernorm_bwd (dx, dg, db +=), but
 * the partial-sum workspace is a fixed array of 8 MiB in the library's device
 * memory (one per GPU, held until the process ends) instead of arena scratch:
 * the call allocates nothing, on the device or through the arena.  A shape
 * whose workspace (tt_layernorm_bwd_workspace) exceeds 8 MiB is TT_EINVAL with
 * nothing enqueued — e.g. up to 16384 rows at C <= 1024 fit.  Every call on a
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race on it; calls ordered on one stream do not
 * (each call writes every partial it reads, so leftover contents are never
 * read).  Its kernels are not timed by tt_ctx_profile. */
int tt_layernorm_bwd_noalloc(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                             const float *mean, const float *rstd, const float *g,
                             const float *dy, float *dx, float *dg, float *db);

/* GELU, tanh form (tinytorch page §3 item 4), elementwise on n values of a
 * mode tensor.  Backward uses the analytic derivative of the tanh form
 * (the page's printed backward is not that derivative): dx = dy * gelu'(x),
 * dx written. */
int tt_gelu_fwd(tt_ctx *ctx, tt_mode mode, size_t n, const void *x, void *y);
int tt_gelu_bwd(tt_ctx *ctx, tt_mode mode, size_t n, const void *x, const void *dy, void *dx);

/* Causal multi-head self-attention — tinytorch page §4 (causal mask, stable
 * softmax); Forge page "最硬的一关" (scale 1/sqrt(d_k), -inf above the
 * diagonal).  qkv [B,T,3C] mode tensor with q | k | v column blocks, head h
 * owning columns h*hs .. h*hs+hs-1 of each; out [B,T,C] mode tensor; lse
 * [B,NH,T] float32 = log of each row's softmax denominator (of the scaled
 * scores).  hs must be 64; T >= 1 (ragged T handled). */
int tt_attn_fwd(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, int hs, const void *qkv,
                void *out, float *lse);
/* Backward: dout [B,T,C] mode tensor -> dqkv [B,T,3C] mode tensor (written).
 * Uses out and lse from the forward.  Scratch comes from the arena. */
int tt_attn_bwd(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, int hs, const void *qkv,
                const void *out, const float *lse, const void *dout, void *dqkv);

/* Fused softmax + cross-entropy, forward and backward in place — tinytorch
 * page §3 item 5 (dlogits = probs - onehot), Forge page "核心组件清单"
 * (cross-entropy fused with log-softmax) and "瓶颈分析是否合理" (one fused
 * pass instead of three).  logits [N, ld] mode tensor, the first V columns
 * used; on return it holds dz = (softmax(z) - onehot(y)) * grad_scale in the
 * first V columns and 0 in columns V..ld-1.  targets [N] int32 in [0,V).
 * loss: one float32 receiving mean_n(logsumexp(z_n) - z_n[y_n]) (written).
 * grad_scale <= 0 means 1/N. */
int tt_ce_fwdbwd(tt_ctx *ctx, tt_mode mode, int N, int V, int ld, void *logits,
                 const int32_t *targets, float *loss, float grad_scale);

/* Token + position embedding — tinytorch page §3 item 6.
 * tok [B,T] int32 in [0,V); wte [V,C], wpe [>=T,C], x0 [B,T,C] float32.
 * x0[b,t] = wte[tok[b,t]] + wpe[t].  Ids outside [0,V) give a NaN row and
 * TT_ERANGE at the next tt_ctx_sync. */
int tt_embed_fwd(tt_ctx *ctx, int B, int T, int C, int V, const int32_t *tok,
                 const float *wte, const float *wpe, float *x0);
/* dwte [V,C] += scatter of dx0 rows by token id; dwpe [>=T,C] += sum over b. */
int tt_embed_bwd(tt_ctx *ctx, int B, int T, int C, int V, const int32_t *tok,
                 const float *dx0, float *dwte, float *dwpe);

/* Optimisers.  AdamW — tinytorch page §3 item 7 (m, v, bias correction with
 * t = step + 1) and Forge page "核心组件清单" (decoupled weight decay):
 *   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   w -= lr * (m/(1-b1^t) / (sqrt(v/(1-b2^t)) + eps) + wd * wd_mult * w).
 * w_lowp (nullable) receives a bf16 copy of the new w.  t is 1-based. */
typedef struct {
  float *w;
  const float *g;
  float *m;
  float *v;
  void *w_lowp;
  size_t n;
  float wd_mult;
} tt_param;
int tt_adamw_step(tt_ctx *ctx, const tt_param *params /* [host] */, int count, float lr,
                  float beta1, float beta2, float eps, float wd, int t);
/* SGD — tinytorch page §8 step 5: w -= lr * g. */
int tt_sgd_step(tt_ctx *ctx, float *w, const float *g, size_t n, float lr);

/* The tiny classifier's whole training step in ONE launch (tinytorch page,
 * section 8 step 5: Linear -> tanh-GELU -> Linear -> softmax cross-entropy,
 * backward, SGD): x [N,I], labels [N] int32 in [0,C), W1 [I,H], b1 [H],
 * W2 [H,C], b2 [C] float32.  loss [1] receives the mean cross-entropy of the
 * step's forward; the weights are updated in place (w -= lr * grad); gW1,
 * gb1, gW2, gb2 (nullable) receive the gradients.  One workgroup holds
 * everything in LDS: N*I + I*H + H + H*C + C + 2*N*H + N*C + N floats must
 * fit in 16384 (TT_EINVAL otherwise).  Labels outside [0,C) give NaN and
 * TT_ERANGE at the next tt_ctx_sync. */
int tt_mlp_step(tt_ctx *ctx, int N, int I, int H, int C, const float *x, const int32_t *labels,
                float *W1, float *b1, float *W2, float *b2, float lr, float *loss, float *gW1,
                float *gb1, float *gW2, float *gb2);
/* float32 -> bf16 (round to nearest even) copy of n values. */
int tt_cast_bf16(tt_ctx *ctx, size_t n, const float *src, void *dst);

/* ------------------------------------------------------------------------ */
/* Composite calls.                                                           */
/* ------------------------------------------------------------------------ */

/* One pre-LN transformer block — tinytorch page §3 item 6:
 *   x1 = x + attn(LN1(x)) ; y = x1 + MLP(LN2(x1)), MLP = fc -> GELU -> fcproj.
 * F is the MLP width (4C for GPT-2); hs = C/NH must be 64. */
typedef struct {
  int B, T, C, NH, F;
  tt_mode mode;
  float ln_eps;
} tt_block_cfg;
/* Weight matrices in the mode dtype ([in,out]); biases and LN params float32. */
typedef struct {
  const float *ln1_g, *ln1_b;
  const void *w_qkv; const float *b_qkv;   /* [C,3C], [3C] */
  const void *w_proj; const float *b_proj; /* [C,C],  [C]  */
  const float *ln2_g, *ln2_b;
  const void *w_fc; const float *b_fc;     /* [C,F],  [F]  */
  const void *w_fcp; const float *b_fcp;   /* [F,C],  [C]  */
} tt_block_w;
/* Gradients, all float32, accumulated (+=). */
typedef struct {
  float *ln1_g, *ln1_b, *w_qkv, *b_qkv, *w_proj, *b_proj;
  float *ln2_g, *ln2_b, *w_fc, *b_fc, *w_fcp, *b_fcp;
} tt_block_g;
/* Activations the backward needs, carved from the arena (opaque).  In the
 * 16-bit modes it also holds transposed copies of the four weight matrices
 * (2 (4C^2 + 2CF) bytes) and the plan of the grouped weight-gradient launch;
 * creation then waits for the stream once. */
typedef struct tt_block_saved tt_block_saved;
int tt_block_saved_create(tt_ctx *ctx, const tt_block_cfg *cfg, tt_block_saved **out);
/* NULL-safe; the device memory returns with the arena. */
void tt_block_saved_destroy(tt_block_saved *saved);
/* x, y [B,T,C] float32.  16-bit modes: the weight matrices are transposed
 * into the saved buffers first (one launch), so the forward products run the
 * same k-major kernels as the whole-model step. */
int tt_block_fwd(tt_ctx *ctx, const tt_block_cfg *cfg, const tt_block_w *w, const float *x,
                 float *y, tt_block_saved *saved);
/* dy [B,T,C] float32 -> dx [B,T,C] float32 (written); grads +=.  Scratch
 * from the arena.  16-bit modes: the four weight gradients run as one
 * grouped launch after the activation gradients (as in the whole-model
 * step); when the scratch or gradient addresses differ from the previous
 * call's, the launch table is re-uploaded and the call waits for the stream. */
int tt_block_bwd(tt_ctx *ctx, const tt_block_cfg *cfg, const tt_block_w *w,
                 const tt_block_saved *saved, const float *dy, float *dx, tt_block_g *g);

/* Tied LM head + mean cross-entropy, forward and backward (tinytorch page §3
 * items 5-6; Forge page "瓶颈分析是否合理").  h [N,C] mode tensor, wte [V,C]
 * mode tensor, targets [N] int32.  loss: one float32 (written, the mean).
 * dh [N,C] float32 (written).  dwte [V,C] float32 (+=).  The [N,V] logits
 * live in arena scratch (mode dtype) and are overwritten by their gradient;
 * in the 16-bit modes the arena also holds wte transposed ([C, V rounded up
 * to 64], one launch) so that dh reads both operands k-major. */
int tt_lmhead_ce_fwdbwd(tt_ctx *ctx, tt_mode mode, int N, int C, int V, const void *h,
                        const void *wte, const int32_t *targets, float *loss, float *dh,
                        float *dwte);

/* Whole GPT-2 model: parameters, gradients, AdamW moments and (TT_BF16) a
 * bf16 shadow of the parameters, all in one arena region; activations for a
 * batch of up to B_max x T_max tokens.  The token table has V_pad >= V rows
 * (rows V..V_pad-1 stay zero) and is tied to the LM head. */
typedef struct {
  int L, C, NH, F, V, V_pad, T_max, B_max;
  tt_mode mode;
  float ln_eps;
} tt_model_cfg;
int tt_model_create(tt_ctx *ctx, const tt_model_cfg *cfg, tt_model **out);
void tt_model_destroy(tt_model *model); /* NULL-safe; memory returns with the arena */
/* Parameter table: count [host] receives the number of tensors; when params
 * [host] is non-NULL it must hold *count entries and receives, in order,
 * wte [V_pad,C], wpe [T_max,C], per layer ln1_g, ln1_b, w_qkv, b_qkv, w_proj,
 * b_proj, ln2_g, ln2_b, w_fc, b_fc, w_fcp, b_fcp, then lnf_g, lnf_b — with
 * device pointers to the master weight (w), gradient (g), moments (m, v) and
 * shadow (w_lowp, NULL in TT_F32).  Callers write initial weights through w
 * and then call tt_model_refresh_shadow. */
int tt_model_param_table(tt_model *model, tt_param *params, int *count);
/* Total float32 parameter slots (including alignment padding). */
int tt_model_num_params(const tt_model *model, size_t *n_slots, size_t *n_params);
/* Recompute the bf16 shadow from the master weights and zero m, v. */
int tt_model_refresh_shadow(tt_model *model);
/* One training step (tinytorch page §3 item 7: forward, zero grads, backward,
 * Adam update), loss on every position with next-token targets, mean over the
 * B*T positions.  tok, targets [B,T] int32.  loss: one float32 (written).
 * nonfinite: nullable int32 device flag.  When given, it is cleared and then
 * set to 1 if the loss or any gradient entry is inf or NaN, and the AdamW
 * update is then dropped: weights, moments and shadows stay bit for bit as
 * they were (the C++/CUDA page, section 5.2, checks for NaN before the
 * optimizer step).  The check reads the whole gradient buffer once (4 bytes
 * per parameter); with NULL there is no check and AdamW always runs.  In
 * TT_FP16 the flag is the loss-scaled step's overflow (tt_model_loss_scale_*).
 * t: 1-based AdamW step.  B <= B_max, T <= T_max. */
int tt_train_step(tt_ctx *ctx, tt_model *model, int B, int T, const int32_t *tok,
                  const int32_t *targets, float lr, float beta1, float beta2, float eps,
                  float wd, int t, float *loss, int32_t *nonfinite);
/* Forward + backward only (gradients written to the model's gradient
 * buffer, zeroed first), no optimizer step. */
int tt_model_fwd_bwd(tt_ctx *ctx, tt_model *model, int B, int T, const int32_t *tok,
                     const int32_t *targets, float *loss);
/* AdamW over every model parameter in one launch (weight decay on all). */
int tt_model_adamw(tt_ctx *ctx, tt_model *model, float lr, float beta1, float beta2,
                   float eps, float wd, int t);

/* Dynamic loss scaling of a TT_FP16 model (C++/CUDA page, section 3.4: fp16
 * activations and gradients with fp32 master weights; the loss is scaled so
 * that small gradients survive in fp16, and the scale adapts).  Every
 * tt_model_fwd_bwd of a TT_FP16 model multiplies the loss gradient by the
 * current scale, so all stored activation gradients carry it, then divides
 * the float32 parameter gradients by it again and flags any inf / NaN.  The
 * next tt_model_adamw (or the update inside tt_train_step) is then dropped,
 * the scale is multiplied by backoff and the clean-step count restarts;
 * after interval consecutive clean steps the scale is multiplied by growth.
 * tt_train_step's nonfinite flag reports the dropped step.  The state lives
 * on the device (no host synchronisation in the step).  Defaults at
 * creation: scale 65536, interval 1000, growth 1.001, backoff 0.5.
 * set: new policy and scale (the counters restart).  get: synchronises with
 * the context's stream and reads the state (host outputs, nullable).
 * TT_EINVAL for a model not in TT_FP16. */
int tt_model_loss_scale_set(tt_ctx *ctx, tt_model *model, float scale, int interval, float growth,
                            float backoff);
int tt_model_loss_scale_get(tt_ctx *ctx, tt_model *model, float *scale, int *good_steps,
                            int *skipped);

/* Global-norm gradient clipping over every parameter gradient of the model
 * (the C++/CUDA page, section 3.2, clips the separately stored gradients by
 * their norm; reading: PyTorch's clip_grad_norm_): norm = sqrt(sum g^2) in
 * float64 over all entries, then g *= max_norm / (norm + 1e-6) when that is
 * below 1.  norm (nullable device float) receives the norm before clipping.
 * Call between tt_model_fwd_bwd and tt_model_adamw.  max_norm > 0. */
int tt_model_clip_grad_norm(tt_ctx *ctx, tt_model *model, float max_norm, float *norm);
/* The same on one gradient buffer g [n] float32 (16-byte aligned). */
int tt_clip_grad_norm(tt_ctx *ctx, float *g, size_t n, float max_norm, float *norm);

/* Checkpoints in the safetensors layout the Forge page reads and writes
 * (section "safetensors格式的安全性优势": 8-byte little-endian header length,
 * JSON header with each tensor's dtype, shape and byte range, raw data).
 * Tensors: the fp32 master weights under the HuggingFace GPT-2 names
 * (wte.weight [V,C], wpe.weight, h.<l>.ln_1.weight, h.<l>.attn.c_attn.weight
 * [C,3C], ..., ln_f.bias; W as [in, out]), the AdamW moments as
 * adam_m.<name> / adam_v.<name>, and step as adam_step (I64 [1]).  save waits
 * for the context's stream and writes path [host string].  load_state reads
 * such a file (a weights-only file, e.g. without adam_* entries, leaves the
 * moments zero; a [V_pad,C] token table is accepted), rebuilds the bf16
 * shadow, and returns the step in *step (nullable; 0 if absent).  Shape or
 * dtype mismatches and I/O errors return TT_EINVAL with the reason in
 * tt_ctx_last_error; after a failed load the model's weights and moments may
 * be partly overwritten (load again before training).  Both synchronise the
 * host with the context's stream. */
int tt_model_save(tt_ctx *ctx, tt_model *model, const char *path, int64_t step);
int tt_model_load_state(tt_ctx *ctx, tt_model *model, const char *path, int64_t *step);

/* ---------------------------------------------------------------- inference
 * Greedy generation with a key/value cache.  The Forge page's GPT-2 inference
 * picks the most likely next token and names the missing KV cache as its main
 * cost (sections "性能瓶颈与未来路线图", "瓶颈分析是否合理"): with causal
 * attention the keys and values of earlier positions do not change, so they
 * are kept and each new token computes only its own.  The result is the same
 * as recomputing the whole sequence (up to rounding order). */

/* Greedy choice: out[n] = index of the largest of logits[n, 0..V-1] (row
 * stride ld >= V, mode dtype), the lowest index on ties and the first NaN if a
 * row holds one.  out [N] int32 (written).  Exact: no rounding is involved. */
int tt_argmax(tt_ctx *ctx, tt_mode mode, int N, int V, int ld, const void *logits,
              int32_t *out);

typedef struct tt_kvcache tt_kvcache;
/* A cache for up to B_max sequences of the model's T_max positions: per
 * layer the keys and values of every processed position ([B_max, T_max, 2C],
 * mode dtype) and the decode step's row buffers, carved from the context's
 * arena (valid until it is reset below them or destroyed).  B_max <= the
 * model's B_max. */
int tt_kvcache_create(tt_ctx *ctx, tt_model *model, int B_max, tt_kvcache **out);
void tt_kvcache_destroy(tt_kvcache *cache); /* NULL-safe */
/* Prefill: the forward of the training step over tok [B,T] int32 (positions
 * 0..T-1), keeping every layer's keys and values in the cache; then the
 * logits of position T-1 and their greedy choice.  logits (nullable) [B,V]
 * mode dtype (written); next [B] int32 (written).  Uses the model's
 * activation buffers (a later training step overwrites them, not the cache).
 * B <= cache B_max, 1 <= T <= T_max. */
int tt_model_prefill(tt_ctx *ctx, tt_model *model, tt_kvcache *cache, int B, int T,
                     const int32_t *tok, void *logits, int32_t *next);
/* Decode one position: tok [B] int32 are the tokens at position pos of the B
 * sequences, whose positions 0..pos-1 are in the cache (pos = the prefill's
 * T for the first call, +1 per call).  Appends position pos to the cache and
 * writes its logits (nullable, [B,V] mode dtype) and greedy choice next [B].
 * pos < T_max. */
int tt_model_decode(tt_ctx *ctx, tt_model *model, tt_kvcache *cache, int B, int pos,
                    const int32_t *tok, void *logits, int32_t *next);

/* ---------------------------------------------------------------- graph
 * Recorded-graph autograd over the library's float32 ops — the tinytorch
 * page, section 3 item 3 (each op's result remembers its op and inputs;
 * Backward walks from the loss to the inputs) with the non-recursive
 * topological walk its comparison table recommends; gradients accumulate
 * with += (C++/CUDA page, section 3.2).  Tensors are 2-D [rows, cols]
 * row-major float32 and named by integer ids in creation order.  A node's
 * inputs precede it, so creation order is topological.  Values and the
 * gradients of computed nodes are carved from the context's arena (valid
 * until it is reset below them or destroyed); leaves use caller memory.
 * Every call validates on the host first (TT_EINVAL on a bad id or shape)
 * and then enqueues kernels on the context's stream. */
typedef struct tt_graph tt_graph;
int tt_graph_create(tt_ctx *ctx, tt_graph **out);
void tt_graph_destroy(tt_graph *graph); /* NULL-safe; arena memory stays */
/* A leaf: data [rows, cols] float32 (caller-owned, read at each forward);
 * grad (nullable) [rows, cols] float32 receiving += dloss/ddata at each
 * backward (NULL: no gradient flows into this leaf).  16-byte aligned. */
int tt_graph_leaf(tt_graph *graph, int rows, int cols, float *data, float *grad, int *id);
/* c = a @ b ([M,K] x [K,N] -> [M,N]); backward dA += dC·bᵀ, dB += aᵀ·dC. */
int tt_graph_matmul(tt_graph *graph, int a, int b, int *id);
/* c = a + b, b of a's shape or one row [1, cols] added to every row (the
 * bias of a linear layer; its gradient is the column sum). */
int tt_graph_add(tt_graph *graph, int a, int b, int *id);
/* c = tanh-form GELU(a) (tinytorch page, section 3 item 4). */
int tt_graph_gelu(tt_graph *graph, int a, int *id);
/* c = softmax of each row of a; backward dA += c∘(dC − rowsum(dC∘c)). */
int tt_graph_softmax(tt_graph *graph, int a, int *id);
/* [1,1] loss = mean over rows of logsumexp(z_r) − z_r[targets[r]] (fused
 * log-softmax cross-entropy, tt_ce_fwdbwd); backward dz += dloss ·
 * (softmax(z) − onehot)/rows.  targets [rows of z] int32 in [0, cols),
 * device, read at each forward. */
int tt_graph_cross_entropy(tt_graph *graph, int logits, const int32_t *targets, int *id);
/* Compute node and every ancestor it needs, in creation order. */
int tt_graph_forward(tt_graph *graph, int node);
/* Seed dloss = 1 and apply every reachable node's gradient rule in reverse
 * creation order, using the values of the last forward.  Gradients of
 * computed nodes restart from zero on each call; leaf gradients accumulate
 * (clear them with tt_graph_zero_grad).  loss: a computed [1,1] node. */
int tt_graph_backward(tt_graph *graph, int loss);
/* Zero every gradient buffer of the graph, the leaves' included. */
int tt_graph_zero_grad(tt_graph *graph);
/* One SGD training step — forward(loss), zero_grad, backward(loss), then
 * w -= lr * grad on every leaf that has a gradient (tinytorch page, section
 * 8: Forward, ZeroGrad, Backward, SGD) — recorded once as a HIP graph, so a
 * step is one launch (tt_graph_step, on the context's stream).  The
 * recording sees the graph's nodes and buffers as they are now: capture
 * again after adding nodes.  Capturing again replaces the previous step.
 * Not while profiling is on. */
int tt_graph_capture_sgd_step(tt_graph *graph, int loss, float lr);
int tt_graph_step(tt_graph *graph);
/* A node's value and gradient (device pointers; grad NULL when no gradient
 * flows through it) and shape; every output nullable. */
int tt_graph_tensor(tt_graph *graph, int id, float **value, float **grad, int *rows, int *cols);

/* ------------------------------------------------------------------------ */
/* Roofline probes (measurement only; the C++/CUDA page, section 2.2, times  */
/* each op with an event pair).  They time, with HIP events on the context's */
/* stream, what the GPU sustains with nothing else in the way; the benchmark */
/* reports kernels against these next to the vendor's peak figures.  Both    */
/* wait for the stream.                                                      */
/* ------------------------------------------------------------------------ */

/* v_mfma_f32_16x16x32_bf16 on register operands only: waves_per_simd (1..8)
 * four-wave workgroups per CU, each wave cycling over `accumulators` (8, 16
 * or 32) independent accumulators for `iters` rounds (<= 2^24).  *tflops
 * [host] receives the dense bf16 rate (2*16*16*32 FLOP per MFMA). */
int tt_probe_mfma(tt_ctx *ctx, int waves_per_simd, int accumulators, int iters, double *tflops);
/* Streaming HBM rate over a caller's device buffer of `bytes` (>= 1 MiB,
 * multiple of 32, 16-byte aligned; its contents are read, and with copy != 0
 * its first half is copied over its second half).  Five passes after one
 * warm-up; *gbs [host] receives bytes read (+ written) per second / 1e9. */
int tt_probe_hbm(tt_ctx *ctx, void *buf, size_t bytes, int copy, double *gbs);
/* Per-CU ceilings, counted in shader clocks (clock64() around each wave's
 * loop: independent of the clock the part runs at).  One workgroup of 8
 * waves per CU (two per SIMD).
 * tt_probe_lds: each wave reads 8 lane-linear 1 KB fragments per round from
 * LDS (ds_read_b128) and, with mfma != 0, issues the 16 MFMAs of a 64 x 64
 * tile on them.  *bytes_per_clk [host]: LDS bytes read per clock per CU;
 * *tflops [host]: the MFMA rate (0 without mfma).
 * tt_probe_lds_load: 16-byte direct-to-LDS loads (buffer_load ... lds), 16 in
 * flight per wave, from a caller's device buffer (64 MiB .. 2 GiB, 16-byte
 * aligned, read only): resident != 0 streams a 64 KB window per workgroup
 * (L2 hits), else 4 MB windows (HBM).  *bytes_per_clk [host]: per CU.
 * tt_probe_issue: 8 independent chains per wave; the first wave of each
 * SIMD runs v_fma_f32 (which = 0, 1), v_exp_f32 (2, 3) or
 * v_mfma_f32_16x16x32_bf16 (4 .. 7); the second wave is idle (0, 2, 4), runs
 * the same (1, 3, 5), FMA (6) or exp (7).  *first, *second [host]: clocks
 * per instruction of each (0 for an idle one). */
int tt_probe_lds(tt_ctx *ctx, int mfma, double *bytes_per_clk, double *tflops);
int tt_probe_lds_load(tt_ctx *ctx, void *buf, size_t bytes, int resident, double *bytes_per_clk);
int tt_probe_issue(tt_ctx *ctx, int which, double *first, double *second);

#ifdef __cplusplus
}
#endif

#endif /* TT_H */
