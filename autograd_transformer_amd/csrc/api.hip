// Host side of the C ABI: argument validation and the op schedule of the
// block, the LM head and the whole training step.  Every step runs in the
// HIP kernels of this library; this file only validates and enqueues.
#include <math.h>
#include <string.h>

#include <vector>

#include "tt_internal.h"

namespace {

inline size_t esize(tt_mode m) { return tt_lowp(m) ? 2 : 4; }
inline bool mode_ok(int m) { return m == TT_F32 || m == TT_BF16 || m == TT_FP16; }

GemmArgs gemm_args() {
  GemmArgs g;
  memset(&g, 0, sizeof g);
  g.split_k = 0;
  return g;
}

// y[M,N] (+)= A[M,K] (k-major, lda) · B where B is W[K,N] row-major (ldb = N),
// i.e. the forward of a linear layer.  Wt, when not NULL, is the same weight
// stored transposed ([N,K], k-major), which the bf16 GEMM reads faster.
int linear_fwd_gemm(tt_ctx *ctx, tt_mode mode, int M, int K, int N, const void *X, int ldx,
                    const void *W, const void *Wt, const float *bias, int epi, void *out,
                    int ldo, bool out_lowp, const float *resid, int ldr, void *aux, int ldaux) {
  GemmArgs g = gemm_args();
  g.A = X; g.lda = ldx; g.a_kmajor = true;
  if (Wt) {
    g.B = Wt; g.ldb = K; g.b_kmajor = true;
  } else {
    g.B = W; g.ldb = N; g.b_kmajor = false;
  }
  g.M = M; g.N = N; g.K = K;
  g.epi = epi; g.out = out; g.ldo = ldo; g.out_bf16 = out_lowp;
  g.bias = bias; g.resid = resid; g.ldr = ldr; g.aux = aux; g.ldx = ldaux;
  return tt_gemm(ctx, mode, g);
}

// dX[M,K] = dY[M,N] · Wᵀ  (W [K,N]), with an epilogue; colsum (nullable)
// accumulates the column sums of the stored dX.
int linear_dx_gemm(tt_ctx *ctx, tt_mode mode, int M, int K, int N, const void *dY, int ldy,
                   const void *W, int epi, void *out, int ldo, bool out_lowp, void *aux,
                   int ldaux, float *colsum = nullptr) {
  GemmArgs g = gemm_args();
  g.A = dY; g.lda = ldy; g.a_kmajor = true;
  g.B = W; g.ldb = N; g.b_kmajor = true;
  g.M = M; g.N = K; g.K = N;
  g.epi = epi; g.out = out; g.ldo = ldo; g.out_bf16 = out_lowp;
  g.aux = aux; g.ldx = ldaux;
  g.colsum = colsum;
  return tt_gemm(ctx, mode, g);
}

// dW[K,N] += Xᵀ · dY  (X [M,K] row-major with ldx, dY [M,N] with ldy); with
// overwrite, dW = Xᵀ · dY.
int linear_dw_gemm(tt_ctx *ctx, tt_mode mode, int M, int K, int N, const void *X, int ldx,
                   const void *dY, int ldy, float *dW, bool overwrite = false) {
  GemmArgs g = gemm_args();
  g.A = X; g.lda = ldx; g.a_kmajor = false;
  g.B = dY; g.ldb = ldy; g.b_kmajor = false;
  g.M = K; g.N = N; g.K = M;
  g.epi = EPI_ACCUM; g.out = dW; g.ldo = N; g.out_bf16 = false;
  g.overwrite = overwrite;
  return tt_gemm(ctx, mode, g);
}

// ------------------------------------------------------------ block pieces

// Transposed bf16 copies of a layer's weight matrices (all NULL: use the
// [K,N] weights).
struct LayerWT {
  const void *w_qkv = nullptr, *w_proj = nullptr, *w_fc = nullptr, *w_fcp = nullptr;
};

struct LayerBufs {
  void *ln1; float *mean1, *rstd1;
  void *qkv; void *att; float *lse;
  float *x1;
  void *ln2; float *mean2, *rstd2;
  void *h; void *g;
};

struct BwdScratch {
  float *dtmp;   // [N,C] f32
  void *datt;    // [N,C] mode
  void *dqkv;    // [N,3C] mode
  void *dh;      // [N,F] mode
  float *Dv;     // [B*NH*T]
};

int alloc_layer(tt_ctx *ctx, tt_mode mode, int N, int C, int F, int B, int NH, int T,
                LayerBufs &s) {
  const size_t es = esize(mode);
  void *p;
#define A_(field, bytes) TT_TRY(tt_arena_alloc(ctx, (bytes), &p)); s.field = (decltype(s.field))p;
  A_(ln1, (size_t)N * C * es)
  A_(mean1, (size_t)N * 4) A_(rstd1, (size_t)N * 4)
  A_(qkv, (size_t)N * 3 * C * es)
  A_(att, (size_t)N * C * es)
  A_(lse, (size_t)B * NH * T * 4)
  A_(x1, (size_t)N * C * 4)
  A_(ln2, (size_t)N * C * es)
  A_(mean2, (size_t)N * 4) A_(rstd2, (size_t)N * 4)
  A_(h, (size_t)N * F * es)
  A_(g, (size_t)N * F * es)
#undef A_
  return TT_OK;
}

int alloc_bwd_scratch(tt_ctx *ctx, tt_mode mode, int N, int C, int F, int B, int NH, int T,
                      BwdScratch &s) {
  const size_t es = esize(mode);
  void *p;
  TT_TRY(tt_arena_alloc(ctx, (size_t)N * C * 4, &p)); s.dtmp = (float *)p;
  TT_TRY(tt_arena_alloc(ctx, (size_t)N * C * es, &p)); s.datt = p;
  TT_TRY(tt_arena_alloc(ctx, (size_t)N * 3 * C * es, &p)); s.dqkv = p;
  TT_TRY(tt_arena_alloc(ctx, (size_t)N * F * es, &p)); s.dh = p;
  TT_TRY(tt_arena_alloc(ctx, (size_t)B * NH * T * 4, &p)); s.Dv = (float *)p;
  return TT_OK;
}

// Pre-LN block forward (tinytorch page §3 item 6).
int layer_fwd(tt_ctx *ctx, tt_mode mode, int B, int T, int C, int NH, int F, float eps,
              const tt_block_w &w, const LayerWT &wt, const float *x, float *y,
              const LayerBufs &s) {
  const int N = B * T;
  const bool lp = tt_lowp(mode);
  TT_TRY(tt_layernorm_fwd_impl(ctx, mode, N, C, eps, x, w.ln1_g, w.ln1_b, s.ln1, s.mean1, s.rstd1));
  TT_TRY(linear_fwd_gemm(ctx, mode, N, C, 3 * C, s.ln1, C, w.w_qkv, wt.w_qkv, w.b_qkv, EPI_STORE, s.qkv,
                         3 * C, lp, nullptr, 0, nullptr, 0));
  TT_TRY(tt_attn_fwd_impl(ctx, mode, B, T, NH, s.qkv, s.att, s.lse));
  TT_TRY(linear_fwd_gemm(ctx, mode, N, C, C, s.att, C, w.w_proj, wt.w_proj, w.b_proj, EPI_RESID, s.x1, C, false,
                         x, C, nullptr, 0));
  TT_TRY(tt_layernorm_fwd_impl(ctx, mode, N, C, eps, s.x1, w.ln2_g, w.ln2_b, s.ln2, s.mean2, s.rstd2));
  TT_TRY(linear_fwd_gemm(ctx, mode, N, C, F, s.ln2, C, w.w_fc, wt.w_fc, w.b_fc, EPI_GELU, s.g, F, lp,
                         nullptr, 0, s.h, F));
  TT_TRY(linear_fwd_gemm(ctx, mode, N, F, C, s.g, F, w.w_fcp, wt.w_fcp, w.b_fcp, EPI_RESID, y, C, false,
                         s.x1, C, nullptr, 0));
  return TT_OK;
}

// Where one block's backward reads and writes its activation gradients.
// rl_in is the GEMM operand copy of the residual gradient on entry (bf16 in
// TT_BF16, the fp32 gradient itself in TT_F32), rl_mid the copy written by the
// LN2 backward, rl_out (nullable in TT_BF16) the copy of the returned
// gradient; dh and dqkv receive the MLP and attention input gradients.  One
// buffer may serve all three copies when nothing reads them later; kept
// apart, they let the weight gradients run after the whole backward.
struct BwdIO {
  void *rl_in, *rl_mid, *rl_out;
  void *dh, *dqkv;
  bool defer_dw;   // leave the four weight-matrix gradients to the caller
  // non-NULL: the LayerNorm backward leaves its column partials here and the
  // caller adds them up later (tt_layernorm_bwd_reduce_batch)
  float *ln2_part = nullptr, *ln1_part = nullptr;
  int part_groups = 0;   // capacity of each partial buffer, in groups
};

// Block backward, in place on the residual gradient R (fp32): on entry R
// holds dL/dy, on return dL/dx.  The bias gradient of the MLP
// down-projection is the column sum of rl_in: computed here when
// fcp_bias_here, else already accumulated by whoever produced R (the
// LayerNorm backward above this block).  dsum_below (nullable) receives the
// column sums of rl_out, i.e. the down-projection bias gradient of the block
// below.  overwrite_dw: the weight-matrix gradients are stored (=) instead of
// accumulated (+=).
int layer_bwd(tt_ctx *ctx, tt_mode mode, int B, int T, int C, int NH, int F,
              const tt_block_w &w, const LayerBufs &s, const float *x, float *R, const BwdIO &io,
              const tt_block_g &gr, const BwdScratch &sc, bool fcp_bias_here, float *dsum_below,
              bool overwrite_dw) {
  const int N = B * T;
  const bool lp = tt_lowp(mode);
  // MLP down-projection: dh = (dy · W_fpᵀ) * gelu'(h), whose column sums are
  // the up-projection's bias gradient; dW_fp += gᵀ dy; db_fp.
  TT_TRY(linear_dx_gemm(ctx, mode, N, F, C, io.rl_in, C, w.w_fcp, EPI_GELU_BWD, io.dh, F, lp, s.h,
                        F, gr.b_fc));
  if (!io.defer_dw)
    TT_TRY(linear_dw_gemm(ctx, mode, N, F, C, s.g, F, io.rl_in, C, gr.w_fcp, overwrite_dw));
  if (fcp_bias_here) TT_TRY(tt_colsum(ctx, mode, N, C, C, io.rl_in, gr.b_fcp));
  // MLP up-projection.
  TT_TRY(linear_dx_gemm(ctx, mode, N, C, F, io.dh, F, w.w_fc, EPI_STORE, sc.dtmp, C, false,
                        nullptr, 0));
  if (!io.defer_dw)
    TT_TRY(linear_dw_gemm(ctx, mode, N, C, F, s.ln2, C, io.dh, F, gr.w_fc, overwrite_dw));
  // LN2 backward + residual: R = R + LN2_bwd(dtmp); its column sums are the
  // attention projection's bias gradient.
  if (io.ln2_part)
    TT_TRY(tt_layernorm_bwd_rows(ctx, mode, N, C, s.x1, s.mean2, s.rstd2, w.ln2_g, sc.dtmp, R, R,
                                 lp ? (bf16_t *)io.rl_mid : nullptr, io.ln2_part, io.part_groups));
  else
    TT_TRY(tt_layernorm_bwd_impl(ctx, mode, N, C, s.x1, s.mean2, s.rstd2, w.ln2_g, sc.dtmp, R, R,
                                 lp ? (bf16_t *)io.rl_mid : nullptr, gr.ln2_g, gr.ln2_b, gr.b_proj));
  // Attention projection.
  TT_TRY(linear_dx_gemm(ctx, mode, N, C, C, io.rl_mid, C, w.w_proj, EPI_STORE, sc.datt, C, lp,
                        nullptr, 0));
  if (!io.defer_dw)
    TT_TRY(linear_dw_gemm(ctx, mode, N, C, C, s.att, C, io.rl_mid, C, gr.w_proj, overwrite_dw));
  // Attention.
  // (its kernels also add the column sums of dqkv into the qkv bias gradient)
  TT_TRY(tt_attn_bwd_impl(ctx, mode, B, T, NH, s.qkv, s.att, s.lse, sc.datt, io.dqkv, sc.Dv,
                          gr.b_qkv));
  // QKV projection.
  TT_TRY(linear_dx_gemm(ctx, mode, N, C, 3 * C, io.dqkv, 3 * C, w.w_qkv, EPI_STORE, sc.dtmp, C,
                        false, nullptr, 0));
  if (!io.defer_dw)
    TT_TRY(linear_dw_gemm(ctx, mode, N, C, 3 * C, s.ln1, C, io.dqkv, 3 * C, gr.w_qkv,
                          overwrite_dw));
  // LN1 backward + residual.
  if (io.ln1_part)
    TT_TRY(tt_layernorm_bwd_rows(ctx, mode, N, C, x, s.mean1, s.rstd1, w.ln1_g, sc.dtmp, R, R,
                                 lp ? (bf16_t *)io.rl_out : nullptr, io.ln1_part, io.part_groups));
  else
    TT_TRY(tt_layernorm_bwd_impl(ctx, mode, N, C, x, s.mean1, s.rstd1, w.ln1_g, sc.dtmp, R, R,
                                 lp ? (bf16_t *)io.rl_out : nullptr, gr.ln1_g, gr.ln1_b,
                                 dsum_below));
  return TT_OK;
}

int check_block_cfg(tt_ctx *ctx, const tt_block_cfg *c) {
  TT_REQUIRE(ctx, c != nullptr, "block: cfg is NULL");
  TT_REQUIRE(ctx, mode_ok(c->mode), "block: bad mode");
  TT_REQUIRE(ctx, c->B > 0 && c->T > 0 && c->C > 0 && c->NH > 0 && c->F > 0, "block: bad shape");
  if (c->C % c->NH != 0 || c->C / c->NH != 64)
    return tt_set_error(ctx, TT_EUNSUPPORTED, "block: head size must be 64 (C=%d NH=%d)", c->C, c->NH);
  TT_REQUIRE(ctx, c->C % 8 == 0 && c->F % 8 == 0 && c->C <= 4096, "block: C, F must be multiples of 8, C <= 4096");
  return TT_OK;
}

}  // namespace

// ------------------------------------------------------------ op level ABI

extern "C" int tt_linear_fwd(tt_ctx *ctx, tt_mode mode, int M, int K, int N, const void *X,
                             const void *W, const float *b, void *Y, int epilogue,
                             const float *resid, void *preact) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "linear_fwd: bad mode");
  TT_REQUIRE(ctx, M > 0 && K > 0 && N > 0, "linear_fwd: bad shape");
  TT_REQUIRE(ctx, X && W && Y, "linear_fwd: NULL operand");
  int epi;
  switch (epilogue) {
    case TT_EPI_NONE: epi = EPI_STORE; break;
    case TT_EPI_GELU: epi = EPI_GELU; break;
    case TT_EPI_RESIDUAL:
      TT_REQUIRE(ctx, resid != nullptr, "linear_fwd: RESIDUAL needs resid");
      epi = EPI_RESID;
      break;
    default: return tt_set_error(ctx, TT_EINVAL, "linear_fwd: bad epilogue %d", epilogue);
  }
  return linear_fwd_gemm(ctx, mode, M, K, N, X, K, W, nullptr, b, epi, Y, N, tt_lowp(mode), resid, N,
                         preact, N);
}

extern "C" int tt_linear_bwd(tt_ctx *ctx, tt_mode mode, int M, int K, int N, const void *X,
                             const void *W, const void *dY, float *dX, float *dW, float *db,
                             int accumulate_dX) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "linear_bwd: bad mode");
  TT_REQUIRE(ctx, M > 0 && K > 0 && N > 0, "linear_bwd: bad shape");
  TT_REQUIRE(ctx, dY != nullptr, "linear_bwd: dY is NULL");
  TT_REQUIRE(ctx, !dX || W, "linear_bwd: dX needs W");
  TT_REQUIRE(ctx, !dW || X, "linear_bwd: dW needs X");
  if (dX)
    TT_TRY(linear_dx_gemm(ctx, mode, M, K, N, dY, N, W, accumulate_dX ? EPI_STORE_ACC : EPI_STORE,
                          dX, K, false, nullptr, 0));
  if (dW) TT_TRY(linear_dw_gemm(ctx, mode, M, K, N, X, K, dY, N, dW));
  if (db) TT_TRY(tt_colsum(ctx, mode, M, N, N, dY, db));
  return TT_OK;
}

extern "C" int tt_layernorm_fwd(tt_ctx *ctx, tt_mode mode, int N, int C, float eps,
                                const float *x, const float *g, const float *b, void *y,
                                float *mean, float *rstd) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "layernorm_fwd: bad mode");
  TT_REQUIRE(ctx, tt_aligned16(x) && tt_aligned16(g) && tt_aligned16(b) && tt_aligned16(y),
             "layernorm_fwd: alignment");
  return tt_layernorm_fwd_impl(ctx, mode, N, C, eps, x, g, b, y, mean, rstd);
}

extern "C" int tt_layernorm_bwd(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                                const float *mean, const float *rstd, const float *g,
                                const float *dy, float *dx, float *dg, float *db) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "layernorm_bwd: bad mode");
  TT_REQUIRE(ctx, tt_aligned16(x) && tt_aligned16(dy) && tt_aligned16(dx) && tt_aligned16(g),
             "layernorm_bwd: alignment");
  return tt_layernorm_bwd_impl(ctx, mode, N, C, x, mean, rstd, g, dy, dx, dx, nullptr, dg, db);
}

extern "C" int tt_attn_fwd(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, int hs,
                           const void *qkv, void *out, float *lse) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "attn_fwd: bad mode");
  if (hs != 64) return tt_set_error(ctx, TT_EUNSUPPORTED, "attn_fwd: head size must be 64");
  TT_REQUIRE(ctx, B > 0 && T > 0 && NH > 0, "attn_fwd: bad shape");
  TT_REQUIRE(ctx, qkv && out && lse && tt_aligned16(qkv) && tt_aligned16(out), "attn_fwd: pointers");
  return tt_attn_fwd_impl(ctx, mode, B, T, NH, qkv, out, lse);
}

extern "C" int tt_attn_bwd(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, int hs,
                           const void *qkv, const void *out, const float *lse, const void *dout,
                           void *dqkv) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "attn_bwd: bad mode");
  if (hs != 64) return tt_set_error(ctx, TT_EUNSUPPORTED, "attn_bwd: head size must be 64");
  TT_REQUIRE(ctx, B > 0 && T > 0 && NH > 0, "attn_bwd: bad shape");
  TT_REQUIRE(ctx, qkv && out && lse && dout && dqkv, "attn_bwd: NULL pointer");
  TT_REQUIRE(ctx, tt_aligned16(qkv) && tt_aligned16(out) && tt_aligned16(dout) && tt_aligned16(dqkv),
             "attn_bwd: alignment");
  tt_scratch_scope scope(ctx);
  void *Dv;
  TT_TRY(tt_arena_alloc(ctx, (size_t)B * NH * T * 4, &Dv));
  return tt_attn_bwd_impl(ctx, mode, B, T, NH, qkv, out, lse, dout, dqkv, (float *)Dv);
}

extern "C" int tt_ce_fwdbwd(tt_ctx *ctx, tt_mode mode, int N, int V, int ld, void *logits,
                            const int32_t *targets, float *loss, float grad_scale) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "ce: bad mode");
  TT_REQUIRE(ctx, N > 0 && V > 0 && ld >= V, "ce: bad shape");
  tt_scratch_scope scope(ctx);
  void *rows;
  TT_TRY(tt_arena_alloc(ctx, (size_t)N * 4, &rows));
  return tt_ce_impl(ctx, mode, N, V, ld, logits, targets, (float *)rows, loss,
                    grad_scale > 0.f ? grad_scale : 1.0f / (float)N);
}

// LM head + CE on an [N, ld] logits scratch buffer (ld >= V, ld % 8 == 0).
// wte_t (nullable): the bf16 token table transposed, [C, V_pad] with
// V_pad >= round_up(V, 8); dh then reads it k-major.  The reduction runs to
// round_up(V, 8): the CE pass writes zeros to the gradient's pad columns, so
// the extra terms vanish.
static int lmhead_ce_core(tt_ctx *ctx, tt_mode mode, int N, int C, int V, int ld, const void *h,
                          const void *wte, const void *wte_t, int V_pad, const int32_t *targets,
                          float *loss, float *dh, float *dwte, void *logits, float *row_loss,
                          bool overwrite_dwte, bool skip_dwte = false,
                          const float *scale_dev = nullptr) {
  const bool lp = tt_lowp(mode);
  GemmArgs g = gemm_args();
  // z = h · wteᵀ
  g.A = h; g.lda = C; g.a_kmajor = true;
  g.B = wte; g.ldb = C; g.b_kmajor = true;
  g.M = N; g.N = V; g.K = C;
  g.epi = EPI_STORE; g.out = logits; g.ldo = ld; g.out_bf16 = lp;
  TT_TRY(tt_gemm(ctx, mode, g));
  // loss and dz = (softmax - onehot)/N in place
  TT_TRY(tt_ce_impl(ctx, mode, N, V, ld, logits, targets, row_loss, loss, 1.0f / (float)N,
                    scale_dev));
  // dh = dz · wte
  g = gemm_args();
  g.A = logits; g.lda = ld; g.a_kmajor = true;
  const int V8 = (V + 7) / 8 * 8;
  if (wte_t && V8 <= V_pad && V8 <= ld) {
    g.B = wte_t; g.ldb = V_pad; g.b_kmajor = true;
    g.M = N; g.N = C; g.K = V8;
  } else {
    g.B = wte; g.ldb = C; g.b_kmajor = false;
    g.M = N; g.N = C; g.K = V;
  }
  g.epi = EPI_STORE; g.out = dh; g.ldo = C; g.out_bf16 = false;
  TT_TRY(tt_gemm(ctx, mode, g));
  if (skip_dwte) return TT_OK;
  // dwte += dzᵀ · h
  g = gemm_args();
  g.A = logits; g.lda = ld; g.a_kmajor = false;
  g.B = h; g.ldb = C; g.b_kmajor = false;
  g.M = V; g.N = C; g.K = N;
  g.epi = EPI_ACCUM; g.out = dwte; g.ldo = C; g.out_bf16 = false;
  g.overwrite = overwrite_dwte;   // rows < V only: the pad rows stay as they are
  return tt_gemm(ctx, mode, g);
}

extern "C" int tt_lmhead_ce_fwdbwd(tt_ctx *ctx, tt_mode mode, int N, int C, int V, const void *h,
                                   const void *wte, const int32_t *targets, float *loss, float *dh,
                                   float *dwte) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode_ok(mode), "lmhead_ce: bad mode");
  TT_REQUIRE(ctx, N > 0 && C > 0 && V > 0 && C % 8 == 0, "lmhead_ce: bad shape");
  TT_REQUIRE(ctx, h && wte && targets && loss && dh && dwte, "lmhead_ce: NULL pointer");
  TT_REQUIRE(ctx, tt_aligned16(h) && tt_aligned16(wte), "lmhead_ce: alignment");
  const int ld = (V + 63) / 64 * 64;
  tt_scratch_scope scope(ctx);
  void *logits, *rows, *wte_t = nullptr;
  TT_TRY(tt_arena_alloc(ctx, (size_t)N * ld * esize(mode), &logits));
  TT_TRY(tt_arena_alloc(ctx, (size_t)N * 4, &rows));
  if (tt_lowp(mode)) {
    // The 16-bit token table transposed, [C, ld] with zero columns V .. ld-1,
    // so that dh = dz · wte reads both operands k-major (the whole-model
    // step's kernels); one launch.
    TT_TRY(tt_arena_alloc(ctx, (size_t)C * ld * 2, &wte_t));
    tt_tdesc_set ts;
    TT_TRY(tt_tdesc_set_add(ts, (const bf16_t *)wte, (bf16_t *)wte_t, V, C, ld));
    TT_TRY(tt_transpose_bf16_set(ctx, ts));
  }
  return lmhead_ce_core(ctx, mode, N, C, V, ld, h, wte, wte_t, ld, targets, loss, dh, dwte,
                        logits, (float *)rows, false);
}

// ------------------------------------------------------------ block ABI

// In TT_BF16 / TT_FP16 the block runs the same kernels as the whole-model
// step: the forward products read transposed 16-bit copies of the four
// weight matrices (rebuilt from the caller's weights on every forward, one
// launch), and the backward leaves its four weight gradients to one grouped
// launch after the activation gradients are done.
struct tt_block_saved {
  uint32_t magic;
  tt_block_cfg cfg;
  LayerBufs s;
  float *xin;  // copy of the block input (LN1's backward needs it)
  bf16_t *wt = nullptr;       // 16-bit modes: Wqkvᵀ [3C,C], Wpᵀ [C,C], Wfcᵀ [F,C], Wfpᵀ [C,F]
  GemmGroup dw;               // 16-bit modes: the four weight-gradient products
  std::vector<GemmGroupEntry> dw_host;   // what dw's device table holds
};

namespace {

// Scratch of one block backward in the 16-bit modes, carved in this order
// from the arena at the reset point, so its addresses repeat from call to
// call (and the grouped-gradient table rarely needs an upload).
struct BlockBwdScratch {
  BwdScratch sc;
  void *rl_in = nullptr, *rl_mid = nullptr;
};

int alloc_block_bwd(tt_ctx *ctx, const tt_block_cfg &c, BlockBwdScratch &b) {
  const int N = c.B * c.T;
  TT_TRY(alloc_bwd_scratch(ctx, c.mode, N, c.C, c.F, c.B, c.NH, c.T, b.sc));
  if (tt_lowp(c.mode)) {
    TT_TRY(tt_arena_alloc(ctx, (size_t)N * c.C * 2, &b.rl_in));
    TT_TRY(tt_arena_alloc(ctx, (size_t)N * c.C * 2, &b.rl_mid));
  }
  return TT_OK;
}

// The four weight-gradient products of a block: dW = Xᵀ · dY.
std::vector<GemmGroupEntry> block_dw_entries(const tt_block_cfg &c, const LayerBufs &s,
                                             const BlockBwdScratch &b, const tt_block_g *g) {
  const int C = c.C, F = c.F;
  std::vector<GemmGroupEntry> ent;
  auto prod = [&](const void *X, int ldx, int rows, const void *dY, int ldy, int cols, float *out) {
    GemmGroupEntry e{};
    e.A = X; e.lda = ldx; e.M = rows;
    e.B = dY; e.ldb = ldy; e.N = cols;
    e.out = out; e.ldo = cols;
    ent.push_back(e);
  };
  prod(s.g, F, F, b.rl_in, C, C, g->w_fcp);
  prod(s.ln2, C, C, b.sc.dh, F, F, g->w_fc);
  prod(s.att, C, C, b.rl_mid, C, C, g->w_proj);
  prod(s.ln1, C, C, b.sc.dqkv, 3 * C, 3 * C, g->w_qkv);
  return ent;
}

}  // namespace

extern "C" int tt_block_saved_create(tt_ctx *ctx, const tt_block_cfg *cfg, tt_block_saved **out) {
  TT_TRY(tt_check_ctx(ctx));
  TT_TRY(check_block_cfg(ctx, cfg));
  TT_REQUIRE(ctx, out != nullptr, "block_saved_create: out is NULL");
  const tt_block_cfg c = *cfg;
  const size_t save = ctx->offset;
  tt_block_saved *sv = new tt_block_saved();
  sv->magic = TT_SAVED_MAGIC;
  sv->cfg = c;
  void *p = nullptr;
  const int N = c.B * c.T;
  int rc = alloc_layer(ctx, c.mode, N, c.C, c.F, c.B, c.NH, c.T, sv->s);
  if (rc == TT_OK) rc = tt_arena_alloc(ctx, (size_t)N * c.C * 4, &p);
  sv->xin = (float *)p;
  if (rc == TT_OK && tt_lowp(c.mode)) {
    rc = tt_arena_alloc(ctx, ((size_t)4 * c.C * c.C + 2 * (size_t)c.C * c.F) * 2, &p);
    sv->wt = (bf16_t *)p;
    if (rc == TT_OK) {
      // Plan the grouped weight gradients once: the device tables persist
      // with the saved buffers, and each backward points the entries at its
      // own scratch and the caller's gradients (the plan needs the shapes
      // only; any aligned address stands in until then, nothing runs on it).
      BlockBwdScratch b;
      b.sc.dh = b.sc.dqkv = b.rl_in = b.rl_mid = sv->xin;
      tt_block_g gdum;
      gdum.w_qkv = gdum.w_proj = gdum.w_fc = gdum.w_fcp = sv->xin;
      sv->dw_host = block_dw_entries(c, sv->s, b, &gdum);
      rc = tt_gemm_group_plan(ctx, sv->dw_host.data(), (int)sv->dw_host.size(), N, &sv->dw,
                              c.mode == TT_FP16);
    }
  }
  if (rc != TT_OK) {
    ctx->offset = save;
    sv->magic = 0;
    delete sv;
    return rc;
  }
  *out = sv;
  return TT_OK;
}

static int check_block_w(tt_ctx *ctx, const tt_block_w *w) {
  TT_REQUIRE(ctx, w != nullptr, "block: weights NULL");
  TT_REQUIRE(ctx, w->ln1_g && w->ln1_b && w->w_qkv && w->b_qkv && w->w_proj && w->b_proj &&
                      w->ln2_g && w->ln2_b && w->w_fc && w->b_fc && w->w_fcp && w->b_fcp,
             "block: a weight pointer is NULL");
  return TT_OK;
}

static int check_saved(tt_ctx *ctx, const tt_block_cfg *cfg, const tt_block_saved *saved,
                       const char *what) {
  if (saved->magic != TT_SAVED_MAGIC) return tt_set_error(ctx, TT_ESTALE, "%s: stale saved", what);
  TT_REQUIRE(ctx, saved->cfg.B == cfg->B && saved->cfg.T == cfg->T && saved->cfg.C == cfg->C &&
                      saved->cfg.NH == cfg->NH && saved->cfg.F == cfg->F &&
                      saved->cfg.mode == cfg->mode,
             "%s: saved buffers were made for another shape", what);
  return TT_OK;
}

extern "C" int tt_block_fwd(tt_ctx *ctx, const tt_block_cfg *cfg, const tt_block_w *w,
                            const float *x, float *y, tt_block_saved *saved) {
  TT_TRY(tt_check_ctx(ctx));
  TT_TRY(check_block_cfg(ctx, cfg));
  TT_TRY(check_block_w(ctx, w));
  TT_REQUIRE(ctx, x && y && saved, "block_fwd: NULL pointer");
  TT_TRY(check_saved(ctx, cfg, saved, "block_fwd"));
  const int C = cfg->C, F = cfg->F;
  hipError_t e = hipMemcpyAsync(saved->xin, x, (size_t)cfg->B * cfg->T * C * 4,
                                hipMemcpyDeviceToDevice, ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "block_fwd copy: %s", hipGetErrorString(e));
  LayerWT wt;
  if (saved->wt) {
    // transposed 16-bit weights: [K, N] -> [N, K], one launch for the four
    bf16_t *q = saved->wt, *pj = q + (size_t)3 * C * C, *fc = pj + (size_t)C * C,
           *fp = fc + (size_t)F * C;
    tt_tdesc_set ts;
    TT_TRY(tt_tdesc_set_add(ts, (const bf16_t *)w->w_qkv, q, C, 3 * C, C));
    TT_TRY(tt_tdesc_set_add(ts, (const bf16_t *)w->w_proj, pj, C, C, C));
    TT_TRY(tt_tdesc_set_add(ts, (const bf16_t *)w->w_fc, fc, C, F, C));
    TT_TRY(tt_tdesc_set_add(ts, (const bf16_t *)w->w_fcp, fp, F, C, F));
    TT_TRY(tt_transpose_bf16_set(ctx, ts));
    wt.w_qkv = q; wt.w_proj = pj; wt.w_fc = fc; wt.w_fcp = fp;
  }
  return layer_fwd(ctx, cfg->mode, cfg->B, cfg->T, C, cfg->NH, F, cfg->ln_eps, *w, wt, saved->xin,
                   y, saved->s);
}

extern "C" int tt_block_bwd(tt_ctx *ctx, const tt_block_cfg *cfg, const tt_block_w *w,
                            const tt_block_saved *saved, const float *dy, float *dx,
                            tt_block_g *g) {
  TT_TRY(tt_check_ctx(ctx));
  TT_TRY(check_block_cfg(ctx, cfg));
  TT_TRY(check_block_w(ctx, w));
  TT_REQUIRE(ctx, saved && dy && dx && g, "block_bwd: NULL pointer");
  TT_TRY(check_saved(ctx, cfg, saved, "block_bwd"));
  TT_REQUIRE(ctx, g->ln1_g && g->ln1_b && g->w_qkv && g->b_qkv && g->w_proj && g->b_proj &&
                      g->ln2_g && g->ln2_b && g->w_fc && g->b_fc && g->w_fcp && g->b_fcp,
             "block_bwd: a gradient pointer is NULL");
  const tt_mode mode = cfg->mode;
  const int N = cfg->B * cfg->T, C = cfg->C;
  const bool lp = tt_lowp(mode);
  tt_scratch_scope scope(ctx);
  BlockBwdScratch b;
  TT_TRY(alloc_block_bwd(ctx, *cfg, b));
  // R = dy (in place on dx from here on)
  if (dx != dy) {
    hipError_t e = hipMemcpyAsync(dx, dy, (size_t)N * C * 4, hipMemcpyDeviceToDevice, ctx->stream);
    if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "block_bwd copy: %s", hipGetErrorString(e));
  }
  if (!lp) {
    const BwdIO io{dx, dx, dx, b.sc.dh, b.sc.dqkv, false};
    return layer_bwd(ctx, mode, cfg->B, cfg->T, C, cfg->NH, cfg->F, *w, saved->s, saved->xin, dx,
                     io, *g, b.sc, true, nullptr, false);
  }
  // 16-bit modes: the activation gradients the weight gradients read stay
  // apart (rl_in: dy's copy; rl_mid: the LN2 backward's output; dh; dqkv),
  // and the four weight gradients run as one grouped launch at the end.
  TT_TRY(tt_cast_f32_bf16(ctx, (size_t)N * C, dx, (bf16_t *)b.rl_in, mode == TT_FP16));
  const BwdIO io{b.rl_in, b.rl_mid, nullptr, b.sc.dh, b.sc.dqkv, true};
  TT_TRY(layer_bwd(ctx, mode, cfg->B, cfg->T, C, cfg->NH, cfg->F, *w, saved->s, saved->xin, dx, io,
                   *g, b.sc, true, nullptr, false));
  tt_block_saved *sv = const_cast<tt_block_saved *>(saved);
  const std::vector<GemmGroupEntry> ent = block_dw_entries(*cfg, saved->s, b, g);
  bool same = ent.size() == sv->dw_host.size();
  for (size_t i = 0; same && i < ent.size(); ++i)
    same = ent[i].A == sv->dw_host[i].A && ent[i].B == sv->dw_host[i].B &&
           ent[i].out == sv->dw_host[i].out;
  if (!same) {
    TT_TRY(tt_gemm_group_update(ctx, sv->dw, ent.data(), (int)ent.size(), N));
    sv->dw_host = ent;
  }
  return tt_gemm_group_run(ctx, sv->dw, N, true);
}

extern "C" void tt_block_saved_destroy(tt_block_saved *saved) {
  if (!saved || saved->magic != TT_SAVED_MAGIC) return;
  saved->magic = 0;
  delete saved;
}

// ------------------------------------------------------------ whole model
// Training loop of the tinytorch page (§3 item 7): forward, zero the
// gradients, backward, Adam update — with the loss on every position and the
// LM head tied to the token table.

struct tt_model {
  uint32_t magic;
  tt_ctx *ctx;
  tt_model_cfg cfg;
  size_t n_slots = 0, n_params = 0;
  size_t small_begin = 0;   // first slot of the accumulated (non-matrix) tensors
  std::vector<size_t> off, numel;
  float *w = nullptr, *g = nullptr, *m = nullptr, *v = nullptr;
  bf16_t *lowp = nullptr;
  // TT_BF16: the weight matrices' bf16 shadows transposed (same slot offsets
  // as lowp), rebuilt from lowp whenever lowp changes.
  bf16_t *lowp_t = nullptr;
  std::vector<tt_tdesc> tdesc;
  tt_tdesc *tdesc_dev = nullptr;
  int t_tiles = 0;
  double t_elems = 0;
  std::vector<LayerBufs> layers;
  std::vector<float *> xs;
  void *lnf = nullptr;
  float *meanf = nullptr, *rstdf = nullptr;
  void *logits = nullptr;
  int ld = 0;
  float *row_loss = nullptr;
  float *R = nullptr;
  void *Rl = nullptr;
  BwdScratch sc;
  // TT_BF16: every layer keeps the activation gradients its weight gradients
  // need (the residual gradient's bf16 copies on entry and after the LN2
  // backward, dh, dqkv), so that all weight-matrix gradients, the token
  // table's included, run as one grouped GEMM after the backward.
  std::vector<BwdIO> lio;
  GemmGroup dw_group;
  // ... and leaves the column partials of its 2L+1 LayerNorm backwards in
  // buffers of their own, added up by one launch after the backward
  float *lnf_part = nullptr;
  LnReduceEntry *ln_table = nullptr;   // device, 2L+1 entries
  int n_ln = 0;
  int ln_part_groups = 0;   // capacity of each partial buffer (every N <= B_max T_max)
  // TT_FP16: dynamic loss scaling (device state; host-side policy)
  tt_loss_scale *ls = nullptr;
  int ls_interval = 1000;
  float ls_growth = 1.001f, ls_backoff = 0.5f;
};

namespace {

enum { P_WTE = 0, P_WPE = 1, P_LAYER0 = 2 };
constexpr int PER_LAYER = 12;
inline int p_lnf_g(const tt_model *md) { return P_LAYER0 + PER_LAYER * md->cfg.L; }

int check_model(tt_model *md) {
  if (!md) return TT_EINVAL;
  if (md->magic != TT_MODEL_MAGIC) return TT_ESTALE;
  return TT_OK;
}

const void *mat(const tt_model *md, int idx) {
  if (tt_lowp(md->cfg.mode)) return md->lowp + md->off[idx];
  return md->w + md->off[idx];
}

const void *mat_t(const tt_model *md, int idx) {
  return md->lowp_t ? (const void *)(md->lowp_t + md->off[idx]) : nullptr;
}

// Rebuild the transposed shadows from lowp (one launch for all matrices).
int refresh_transposed(tt_model *md) {
  if (!md->lowp_t) return TT_OK;
  return tt_transpose_bf16(md->ctx, md->tdesc_dev, (int)md->tdesc.size(), md->t_tiles,
                           md->t_elems);
}

void layer_views(const tt_model *md, int l, tt_block_w &w, LayerWT &wt, tt_block_g &gr) {
  const int b = P_LAYER0 + PER_LAYER * l;
  wt.w_qkv = mat_t(md, b + 2); wt.w_proj = mat_t(md, b + 4);
  wt.w_fc = mat_t(md, b + 8); wt.w_fcp = mat_t(md, b + 10);
  auto W = [&](int i) { return (const float *)(md->w + md->off[b + i]); };
  auto G = [&](int i) { return md->g + md->off[b + i]; };
  w.ln1_g = W(0); w.ln1_b = W(1); w.w_qkv = mat(md, b + 2); w.b_qkv = W(3);
  w.w_proj = mat(md, b + 4); w.b_proj = W(5); w.ln2_g = W(6); w.ln2_b = W(7);
  w.w_fc = mat(md, b + 8); w.b_fc = W(9); w.w_fcp = mat(md, b + 10); w.b_fcp = W(11);
  gr.ln1_g = G(0); gr.ln1_b = G(1); gr.w_qkv = G(2); gr.b_qkv = G(3);
  gr.w_proj = G(4); gr.b_proj = G(5); gr.ln2_g = G(6); gr.ln2_b = G(7);
  gr.w_fc = G(8); gr.b_fc = G(9); gr.w_fcp = G(10); gr.b_fcp = G(11);
}

}  // namespace

extern "C" int tt_model_create(tt_ctx *ctx, const tt_model_cfg *cfg, tt_model **out) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, cfg && out, "model_create: NULL argument");
  *out = nullptr;
  const tt_model_cfg c = *cfg;
  TT_REQUIRE(ctx, mode_ok(c.mode), "model_create: bad mode");
  TT_REQUIRE(ctx, c.L > 0 && c.C > 0 && c.NH > 0 && c.F > 0 && c.V > 0 && c.V_pad >= c.V &&
                      c.T_max > 0 && c.B_max > 0,
             "model_create: bad shape");
  if (c.C / c.NH != 64 || c.C % c.NH)
    return tt_set_error(ctx, TT_EUNSUPPORTED, "model_create: head size must be 64");
  TT_REQUIRE(ctx, c.C % 8 == 0 && c.F % 8 == 0 && c.C <= 4096, "model_create: C, F multiples of 8");
  tt_model *md = new tt_model();
  md->magic = TT_MODEL_MAGIC;
  md->ctx = ctx;
  md->cfg = c;
  // Slots: the weight matrices first (each gradient is written whole by one
  // GEMM per step), then every other tensor in one contiguous region (their
  // gradients accumulate and are cleared each step with one fill).  Tensor
  // indices keep the documented order.
  std::vector<bool> whole;
  auto add = [&](size_t n, bool w) {
    md->numel.push_back(n);
    whole.push_back(w);
    md->n_params += n;
  };
  const size_t C = c.C, F = c.F;
  add((size_t)c.V_pad * C, true);
  add((size_t)c.T_max * C, false);
  for (int l = 0; l < c.L; ++l) {
    add(C, false); add(C, false); add(C * 3 * C, true); add(3 * C, false); add(C * C, true);
    add(C, false); add(C, false); add(C, false); add(C * F, true); add(F, false); add(F * C, true);
    add(C, false);
  }
  add(C, false); add(C, false);
  md->off.assign(md->numel.size(), 0);
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) md->small_begin = md->n_slots;
    for (size_t i = 0; i < md->numel.size(); ++i)
      if (whole[i] == (pass == 0)) {
        md->off[i] = md->n_slots;
        md->n_slots += (md->numel[i] + 63) / 64 * 64;  // 256-byte aligned tensors
      }
  }
  const size_t save = ctx->offset;
  int rc = TT_OK;
  void *p;
  auto alloc = [&](size_t bytes) -> void * {
    if (rc != TT_OK) return nullptr;
    rc = tt_arena_alloc(ctx, bytes, &p);
    return rc == TT_OK ? p : nullptr;
  };
  md->w = (float *)alloc(md->n_slots * 4);
  md->g = (float *)alloc(md->n_slots * 4);
  md->m = (float *)alloc(md->n_slots * 4);
  md->v = (float *)alloc(md->n_slots * 4);
  if (tt_lowp(c.mode)) {
    md->lowp = (bf16_t *)alloc(md->n_slots * 2);
    md->lowp_t = (bf16_t *)alloc(md->n_slots * 2);
    // transpose table: wte [V_pad, C], then per layer qkv, proj, fc, fcproj
    auto addt = [&](int idx, int rows, int cols) {
      tt_tdesc d;
      d.src = md->lowp ? md->lowp + md->off[idx] : nullptr;
      d.dst = md->lowp_t ? md->lowp_t + md->off[idx] : nullptr;
      d.rows = rows; d.cols = cols; d.pad_rows = rows;
      d.tiles_c = (cols + 63) / 64; d.tile0 = md->t_tiles;
      md->tdesc.push_back(d);
      md->t_tiles += ((rows + 63) / 64) * d.tiles_c;
      md->t_elems += (double)rows * cols;
    };
    addt(P_WTE, c.V_pad, c.C);
    for (int l = 0; l < c.L; ++l) {
      const int b = P_LAYER0 + PER_LAYER * l;
      addt(b + 2, c.C, 3 * c.C); addt(b + 4, c.C, c.C);
      addt(b + 8, c.C, c.F); addt(b + 10, c.F, c.C);
    }
    md->tdesc_dev = (tt_tdesc *)alloc(md->tdesc.size() * sizeof(tt_tdesc));
    if (rc == TT_OK) {
      hipError_t e = hipMemcpyAsync(md->tdesc_dev, md->tdesc.data(),
                                    md->tdesc.size() * sizeof(tt_tdesc), hipMemcpyHostToDevice,
                                    ctx->stream);
      if (e != hipSuccess) rc = tt_set_error(ctx, TT_EHIP, "model_create copy: %s", hipGetErrorString(e));
    }
  }
  const int N = c.B_max * c.T_max;
  const size_t es = esize(c.mode);
  md->layers.resize(c.L);
  for (int l = 0; l < c.L && rc == TT_OK; ++l)
    rc = alloc_layer(ctx, c.mode, N, c.C, c.F, c.B_max, c.NH, c.T_max, md->layers[l]);
  for (int l = 0; l <= c.L; ++l) md->xs.push_back((float *)alloc((size_t)N * C * 4));
  md->lnf = alloc((size_t)N * C * es);
  md->meanf = (float *)alloc((size_t)N * 4);
  md->rstdf = (float *)alloc((size_t)N * 4);
  md->ld = (c.V + 63) / 64 * 64;
  md->logits = alloc((size_t)N * md->ld * es);
  md->row_loss = (float *)alloc((size_t)N * 4);
  md->R = (float *)alloc((size_t)N * C * 4);
  md->Rl = tt_lowp(c.mode) ? alloc((size_t)N * C * 2) : (void *)md->R;
  if (c.mode == TT_FP16) md->ls = (tt_loss_scale *)alloc(sizeof(tt_loss_scale));
  if (rc == TT_OK) rc = alloc_bwd_scratch(ctx, c.mode, N, c.C, c.F, c.B_max, c.NH, c.T_max, md->sc);
  if (rc == TT_OK && tt_lowp(c.mode)) {
    md->lio.resize(c.L);
    for (int l = 0; l < c.L; ++l) {
      BwdIO &io = md->lio[l];
      io.rl_in = alloc((size_t)N * C * 2);
      io.rl_mid = alloc((size_t)N * C * 2);
      io.dh = alloc((size_t)N * F * 2);
      io.dqkv = alloc((size_t)N * 3 * C * 2);
      io.defer_dw = true;
    }
    for (int l = 0; l < c.L; ++l) md->lio[l].rl_out = l > 0 ? md->lio[l - 1].rl_in : nullptr;
    // The grouped weight-gradient products: dW = Xᵀ · dY with both operands
    // token-major.  Token table first (the largest product), then the layers.
    std::vector<GemmGroupEntry> ent;
    auto prod = [&](const void *X, int ldx, int rows, const void *dY, int ldy, int cols, float *out) {
      GemmGroupEntry e{};
      e.A = X; e.lda = ldx; e.M = rows;
      e.B = dY; e.ldb = ldy; e.N = cols;
      e.out = out; e.ldo = cols;
      ent.push_back(e);
    };
    if (rc == TT_OK) {
      prod(md->logits, md->ld, c.V, md->lnf, c.C, c.C, md->g + md->off[P_WTE]);
      for (int l = c.L - 1; l >= 0; --l) {
        const int b = P_LAYER0 + PER_LAYER * l;
        const LayerBufs &s = md->layers[l];
        const BwdIO &io = md->lio[l];
        prod(s.g, c.F, c.F, io.rl_in, c.C, c.C, md->g + md->off[b + 10]);
        prod(s.ln2, c.C, c.C, io.dh, c.F, c.F, md->g + md->off[b + 8]);
        prod(s.att, c.C, c.C, io.rl_mid, c.C, c.C, md->g + md->off[b + 4]);
        prod(s.ln1, c.C, c.C, io.dqkv, 3 * c.C, 3 * c.C, md->g + md->off[b + 2]);
      }
      rc = tt_gemm_group_plan(ctx, ent.data(), (int)ent.size(), N, &md->dw_group,
                              c.mode == TT_FP16);
    }
    // LayerNorm partials: LN_f, then each layer's LN2 and LN1 from the top
    // (the order the backward runs them; the table's order does not matter).
    // sized for every step shape up to the capacity: the group count is not
    // monotone in the number of rows
    md->ln_part_groups = tt_layernorm_bwd_groups_max(N, c.C);
    const size_t part_floats = (size_t)md->ln_part_groups * 3 * c.C;
    std::vector<LnReduceEntry> lt;
    const int lf = p_lnf_g(md);
    md->lnf_part = (float *)alloc(part_floats * 4);
    lt.push_back({md->lnf_part, md->g + md->off[lf], md->g + md->off[lf + 1],
                  md->g + md->off[P_LAYER0 + PER_LAYER * (c.L - 1) + 11]});
    for (int l = c.L - 1; l >= 0; --l) {
      const int b = P_LAYER0 + PER_LAYER * l;
      BwdIO &io = md->lio[l];
      io.ln2_part = (float *)alloc(part_floats * 4);
      io.ln1_part = (float *)alloc(part_floats * 4);
      io.part_groups = md->ln_part_groups;
      // LN2: gamma, beta, and the projection bias (column sums of its output)
      lt.push_back({io.ln2_part, md->g + md->off[b + 6], md->g + md->off[b + 7],
                    md->g + md->off[b + 5]});
      // LN1: gamma, beta, and the down-projection bias of the block below
      lt.push_back({io.ln1_part, md->g + md->off[b + 0], md->g + md->off[b + 1],
                    l > 0 ? md->g + md->off[b - PER_LAYER + 11] : nullptr});
    }
    md->ln_table = (LnReduceEntry *)alloc(lt.size() * sizeof(LnReduceEntry));
    md->n_ln = (int)lt.size();
    if (rc == TT_OK) {
      const hipError_t e1 = hipMemcpyAsync(md->ln_table, lt.data(), lt.size() * sizeof(LnReduceEntry),
                                           hipMemcpyHostToDevice, ctx->stream);
      // the host vector dies here: make sure the copy has read it
      const hipError_t e2 = e1 == hipSuccess ? hipStreamSynchronize(ctx->stream) : e1;
      if (e2 != hipSuccess) rc = tt_set_error(ctx, TT_EHIP, "model_create: %s", hipGetErrorString(e2));
    }
  }
  for (float *buf : {md->w, md->g, md->m, md->v})
    if (rc == TT_OK) rc = tt_fill_f32(ctx, buf, md->n_slots, 0.f);
  if (rc == TT_OK && md->lowp)
    rc = tt_cast_f32_bf16(ctx, md->n_slots, md->w, md->lowp, c.mode == TT_FP16);
  if (rc == TT_OK) rc = refresh_transposed(md);
  if (rc == TT_OK && md->ls) rc = tt_loss_scale_set(ctx, md->ls, 65536.f);
  if (rc != TT_OK) {
    ctx->offset = save;
    md->magic = 0;
    delete md;
    return rc;
  }
  *out = md;
  return TT_OK;
}

extern "C" void tt_model_destroy(tt_model *model) {
  if (!model || model->magic != TT_MODEL_MAGIC) return;
  model->magic = 0;
  delete model;
}

extern "C" int tt_model_param_table(tt_model *md, tt_param *params, int *count) {
  TT_TRY(check_model(md));
  if (!count) return TT_EINVAL;
  const int n = (int)md->off.size();
  if (params) {
    if (*count < n) return TT_EINVAL;
    for (int i = 0; i < n; ++i) {
      params[i].w = md->w + md->off[i];
      params[i].g = md->g + md->off[i];
      params[i].m = md->m + md->off[i];
      params[i].v = md->v + md->off[i];
      params[i].w_lowp = md->lowp ? (void *)(md->lowp + md->off[i]) : nullptr;
      params[i].n = md->numel[i];
      params[i].wd_mult = 1.0f;
    }
  }
  *count = n;
  return TT_OK;
}

extern "C" int tt_model_num_params(const tt_model *md, size_t *n_slots, size_t *n_params) {
  if (!md) return TT_EINVAL;
  if (md->magic != TT_MODEL_MAGIC) return TT_ESTALE;
  if (n_slots) *n_slots = md->n_slots;
  if (n_params) *n_params = md->n_params;
  return TT_OK;
}

extern "C" int tt_model_refresh_shadow(tt_model *md) {
  TT_TRY(check_model(md));
  tt_ctx *ctx = md->ctx;
  if (md->lowp) TT_TRY(tt_cast_f32_bf16(ctx, md->n_slots, md->w, md->lowp, md->cfg.mode == TT_FP16));
  TT_TRY(refresh_transposed(md));
  TT_TRY(tt_fill_f32(ctx, md->m, md->n_slots, 0.f));
  return tt_fill_f32(ctx, md->v, md->n_slots, 0.f);
}

extern "C" int tt_model_fwd_bwd(tt_ctx *ctx, tt_model *md, int B, int T, const int32_t *tok,
                                const int32_t *targets, float *loss) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "fwd_bwd: bad model handle");
  TT_REQUIRE(ctx, md->ctx == ctx, "fwd_bwd: model belongs to another context");
  const tt_model_cfg &c = md->cfg;
  TT_REQUIRE(ctx, B > 0 && T > 0 && B <= c.B_max && T <= c.T_max, "fwd_bwd: B, T exceed capacity");
  TT_REQUIRE(ctx, tok && targets && loss, "fwd_bwd: NULL pointer");
  const tt_mode mode = c.mode;
  const int N = B * T, C = c.C;
  const bool lp = tt_lowp(mode);

  // Matrix gradients are overwritten by their GEMMs; clear the rest.  (The
  // token table's pad rows are never written and stay zero from creation.)
  TT_TRY(tt_fill_f32(ctx, md->g + md->small_begin, md->n_slots - md->small_begin, 0.f));
  // TT_FP16: this step's overflow flag starts clear (its bits are float 0)
  if (md->ls) TT_TRY(tt_fill_f32(ctx, (float *)&md->ls->overflow, 1, 0.f));
  TT_TRY(tt_embed_fwd(ctx, B, T, C, c.V, tok, md->w + md->off[P_WTE], md->w + md->off[P_WPE],
                      md->xs[0]));
  tt_block_w w;
  LayerWT wt;
  tt_block_g gr;
  for (int l = 0; l < c.L; ++l) {
    layer_views(md, l, w, wt, gr);
    TT_TRY(layer_fwd(ctx, mode, B, T, C, c.NH, c.F, c.ln_eps, w, wt, md->xs[l], md->xs[l + 1],
                     md->layers[l]));
  }
  const int lf = p_lnf_g(md);
  TT_TRY(tt_layernorm_fwd_impl(ctx, mode, N, C, c.ln_eps, md->xs[c.L], md->w + md->off[lf],
                               md->w + md->off[lf + 1], md->lnf, md->meanf, md->rstdf));
  const bool grouped = !md->lio.empty();
  TT_TRY(lmhead_ce_core(ctx, mode, N, C, c.V, md->ld, md->lnf, mat(md, P_WTE), mat_t(md, P_WTE),
                        c.V_pad, targets, loss, md->sc.dtmp, md->g + md->off[P_WTE], md->logits,
                        md->row_loss, true, grouped, md->ls ? &md->ls->scale : nullptr));
  // Each LayerNorm backward also sums its output's columns into the
  // down-projection bias gradient of the block below it.
  auto fcp_bias = [&](int l) { return md->g + md->off[P_LAYER0 + PER_LAYER * l + 11]; };
  void *rl_top = grouped ? md->lio[c.L - 1].rl_in : md->Rl;
  if (grouped)
    TT_TRY(tt_layernorm_bwd_rows(ctx, mode, N, C, md->xs[c.L], md->meanf, md->rstdf,
                                 md->w + md->off[lf], md->sc.dtmp, nullptr, md->R,
                                 lp ? (bf16_t *)rl_top : nullptr, md->lnf_part, md->ln_part_groups));
  else
    TT_TRY(tt_layernorm_bwd_impl(ctx, mode, N, C, md->xs[c.L], md->meanf, md->rstdf,
                                 md->w + md->off[lf], md->sc.dtmp, nullptr, md->R,
                                 lp ? (bf16_t *)rl_top : nullptr, md->g + md->off[lf],
                                 md->g + md->off[lf + 1], fcp_bias(c.L - 1)));
  for (int l = c.L - 1; l >= 0; --l) {
    layer_views(md, l, w, wt, gr);
    const BwdIO io = grouped ? md->lio[l]
                             : BwdIO{md->Rl, md->Rl, md->Rl, md->sc.dh, md->sc.dqkv, false};
    TT_TRY(layer_bwd(ctx, mode, B, T, C, c.NH, c.F, w, md->layers[l], md->xs[l], md->R, io, gr,
                     md->sc, false, l > 0 ? fcp_bias(l - 1) : nullptr, true));
  }
  // Every weight-matrix gradient (stored, not accumulated) in one launch, the
  // LayerNorm parameter and the projection bias gradients in another; then
  // the token rows of the embedding add into the token table's.
  if (grouped) {
    TT_TRY(tt_gemm_group_run(ctx, md->dw_group, N));
    TT_TRY(tt_layernorm_bwd_reduce_batch(ctx, N, C, md->ln_table, md->n_ln));
  }
  TT_TRY(tt_embed_bwd(ctx, B, T, C, c.V, tok, md->R, md->g + md->off[P_WTE],
                      md->g + md->off[P_WPE]));
  // TT_FP16: the gradients carry the loss scale; divide it out and flag
  // overflow (the update is then dropped and the scale halved)
  if (md->ls) TT_TRY(tt_unscale_check(ctx, md->g, md->n_slots, md->ls));
  return TT_OK;
}

// skip (nullable, device): a nonzero flag drops the update (weights,
// moments and both shadows stay as they are).
static int model_adamw(tt_ctx *ctx, tt_model *md, float lr, float beta1, float beta2, float eps,
                       float wd, int t, int32_t *overflow_out, const int32_t *skip = nullptr) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "adamw: bad model handle");
  TT_REQUIRE(ctx, t >= 1, "adamw: t is 1-based");
  const bool f16 = md->cfg.mode == TT_FP16;
  if (md->ls) skip = &md->ls->overflow;
  TT_TRY(tt_adamw_flat(ctx, md->w, md->g, md->m, md->v, md->lowp, md->n_slots, lr, beta1, beta2,
                       eps, wd, t, f16, skip));
  // (a dropped update leaves lowp unchanged, so the rebuilt transposed
  // shadow is unchanged too)
  TT_TRY(refresh_transposed(md));
  if (md->ls)
    TT_TRY(tt_loss_scale_update(ctx, md->ls, md->ls_interval, md->ls_growth, md->ls_backoff,
                                overflow_out));
  return TT_OK;
}

extern "C" int tt_model_adamw(tt_ctx *ctx, tt_model *md, float lr, float beta1, float beta2,
                              float eps, float wd, int t) {
  return model_adamw(ctx, md, lr, beta1, beta2, eps, wd, t, nullptr);
}

extern "C" int tt_train_step(tt_ctx *ctx, tt_model *md, int B, int T, const int32_t *tok,
                             const int32_t *targets, float lr, float beta1, float beta2, float eps,
                             float wd, int t, float *loss, int32_t *nonfinite) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, t >= 1, "train_step: t is 1-based");
  TT_TRY(tt_model_fwd_bwd(ctx, md, B, T, tok, targets, loss));
  if (md->ls)   // TT_FP16: the flag is the step's gradient overflow (update dropped)
    return model_adamw(ctx, md, lr, beta1, beta2, eps, wd, t, nonfinite);
  if (!nonfinite) return model_adamw(ctx, md, lr, beta1, beta2, eps, wd, t, nullptr);
  // The C++/CUDA page (section 5.2) checks for NaN before the optimizer step:
  // the flag is raised by an inf / NaN in the loss or in any gradient, and
  // AdamW then leaves weights, moments and shadows as they were.
  TT_TRY(tt_fill_f32(ctx, (float *)nonfinite, 1, 0.f));
  TT_TRY(tt_check_finite(ctx, loss, 1, nonfinite));
  TT_TRY(tt_check_finite(ctx, md->g, md->n_slots, nonfinite));
  return model_adamw(ctx, md, lr, beta1, beta2, eps, wd, t, nullptr, nonfinite);
}

extern "C" int tt_model_loss_scale_set(tt_ctx *ctx, tt_model *md, float scale, int interval,
                                       float growth, float backoff) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "loss_scale_set: bad model handle");
  TT_REQUIRE(ctx, md->ls != nullptr, "loss_scale_set: the model is not in TT_FP16 mode");
  TT_REQUIRE(ctx, scale > 0.f && interval > 0 && growth >= 1.f && backoff > 0.f && backoff < 1.f,
             "loss_scale_set: need scale > 0, interval > 0, growth >= 1, 0 < backoff < 1");
  md->ls_interval = interval;
  md->ls_growth = growth;
  md->ls_backoff = backoff;
  return tt_loss_scale_set(ctx, md->ls, scale);
}

extern "C" int tt_model_loss_scale_get(tt_ctx *ctx, tt_model *md, float *scale, int *good_steps,
                                       int *skipped) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "loss_scale_get: bad model handle");
  TT_REQUIRE(ctx, md->ls != nullptr, "loss_scale_get: the model is not in TT_FP16 mode");
  tt_loss_scale st;
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e == hipSuccess) e = hipMemcpy(&st, md->ls, sizeof st, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "loss_scale_get: %s", hipGetErrorString(e));
  if (scale) *scale = st.scale;
  if (good_steps) *good_steps = st.good;
  if (skipped) *skipped = st.skipped;
  return TT_OK;
}

// ------------------------------------------------------------ inference
// Greedy generation with a key/value cache (the Forge page's inference loop
// with the cache its sections "性能瓶颈与未来路线图" / "瓶颈分析是否合理"
// call for): a prefill runs the training forward over the prompt and keeps
// every layer's keys and values; each decode step then pushes one token per
// sequence through the same ops on single rows and attends over the cache.

struct tt_kvcache {
  uint32_t magic;
  tt_ctx *ctx;
  tt_model *md;
  int B_max, T_max;
  std::vector<void *> kv;   // per layer [B_max, T_max, 2C], mode dtype
  // decode step rows
  float *x = nullptr, *x1 = nullptr, *mean = nullptr, *rstd = nullptr;
  void *ln = nullptr, *qkv = nullptr, *att = nullptr, *h = nullptr, *g = nullptr;
  void *logits = nullptr;   // [B_max, md->ld]
  float *part = nullptr;    // attention partials [B_max * NH * TT_DECODE_MAX_SPLITS * 66]
  // The step reads its position and tokens from, and writes its choice to,
  // device memory, so one captured graph of the step serves every position.
  int32_t *pos_dev = nullptr, *tok_dev = nullptr, *next_dev = nullptr;
  hipStream_t cap = nullptr;        // capture only (nothing runs on it)
  hipGraphExec_t graph = nullptr;   // the captured step for graph_B sequences
  int graph_B = 0;
};

extern "C" int tt_kvcache_create(tt_ctx *ctx, tt_model *md, int B_max, tt_kvcache **out) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, out != nullptr, "kvcache_create: out is NULL");
  *out = nullptr;
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "kvcache_create: bad model handle");
  TT_REQUIRE(ctx, md->ctx == ctx, "kvcache_create: model belongs to another context");
  const tt_model_cfg &c = md->cfg;
  if (c.mode == TT_FP16)
    return tt_set_error(ctx, TT_EUNSUPPORTED, "kvcache_create: decoding runs in TT_F32 or TT_BF16");
  TT_REQUIRE(ctx, B_max > 0 && B_max <= c.B_max, "kvcache_create: B_max must be in [1, %d]",
             c.B_max);
  if (c.T_max > 16384)
    return tt_set_error(ctx, TT_EUNSUPPORTED, "kvcache_create: T_max above 16384");
  const size_t es = esize(c.mode), C = c.C, F = c.F, B = B_max;
  tt_kvcache *kc = new tt_kvcache();
  kc->magic = TT_KV_MAGIC;
  kc->ctx = ctx;
  kc->md = md;
  kc->B_max = B_max;
  kc->T_max = c.T_max;
  const size_t save = ctx->offset;
  void *p;
  auto alloc = [&](size_t bytes) -> void * {
    if (rc != TT_OK) return nullptr;
    rc = tt_arena_alloc(ctx, bytes, &p);
    return rc == TT_OK ? p : nullptr;
  };
  for (int l = 0; l < c.L; ++l) kc->kv.push_back(alloc(B * c.T_max * 2 * C * es));
  kc->x = (float *)alloc(B * C * 4);
  kc->x1 = (float *)alloc(B * C * 4);
  kc->mean = (float *)alloc(B * 4);
  kc->rstd = (float *)alloc(B * 4);
  kc->ln = alloc(B * C * es);
  kc->qkv = alloc(B * 3 * C * es);
  kc->att = alloc(B * C * es);
  kc->h = alloc(B * F * es);
  kc->g = alloc(B * F * es);
  kc->logits = alloc(B * (size_t)md->ld * es);
  kc->part = (float *)alloc(B * c.NH * (size_t)TT_DECODE_MAX_SPLITS * 66 * 4);
  kc->pos_dev = (int32_t *)alloc(4);
  kc->tok_dev = (int32_t *)alloc(B * 4);
  kc->next_dev = (int32_t *)alloc(B * 4);
  if (rc == TT_OK && hipStreamCreateWithFlags(&kc->cap, hipStreamNonBlocking) != hipSuccess) {
    (void)hipGetLastError();
    rc = tt_set_error(ctx, TT_EHIP, "kvcache_create: stream creation failed");
  }
  if (rc != TT_OK) {
    ctx->offset = save;
    kc->magic = 0;
    delete kc;
    return rc;
  }
  *out = kc;
  return TT_OK;
}

extern "C" void tt_kvcache_destroy(tt_kvcache *kc) {
  if (!kc || kc->magic != TT_KV_MAGIC) return;
  kc->magic = 0;
  (void)hipStreamSynchronize(kc->ctx->stream);
  if (kc->graph) (void)hipGraphExecDestroy(kc->graph);
  if (kc->cap) (void)hipStreamDestroy(kc->cap);
  delete kc;
}

namespace {

int check_kv(tt_ctx *ctx, tt_model *md, tt_kvcache *kc, int B, const void *tok, int32_t *next) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "decode: bad model handle");
  if (!kc || kc->magic != TT_KV_MAGIC) return tt_set_error(ctx, TT_ESTALE, "decode: stale cache");
  TT_REQUIRE(ctx, md->ctx == ctx && kc->md == md, "decode: cache, model and context do not match");
  TT_REQUIRE(ctx, B > 0 && B <= kc->B_max, "decode: B must be in [1, %d]", kc->B_max);
  TT_REQUIRE(ctx, tok && next, "decode: NULL pointer");
  return TT_OK;
}

// Logits of B rows of the final LayerNorm output (row stride ldf elements)
// against the tied token table into the cache's [B, ld] buffer, and their
// greedy choice.
int logits_and_choice(tt_ctx *ctx, tt_model *md, tt_kvcache *kc, int B, const void *f, int ldf,
                      int32_t *next) {
  const tt_model_cfg &c = md->cfg;
  GemmArgs g = gemm_args();
  g.A = f; g.lda = ldf; g.a_kmajor = true;
  g.B = mat(md, P_WTE); g.ldb = c.C; g.b_kmajor = true;
  g.M = B; g.N = c.V; g.K = c.C;
  g.epi = EPI_STORE; g.out = kc->logits; g.ldo = md->ld; g.out_bf16 = c.mode == TT_BF16;
  TT_TRY(tt_gemm(ctx, c.mode, g));
  return tt_argmax(ctx, c.mode, B, c.V, md->ld, kc->logits, next);
}

// (nullable) copy of the cache's logits as [B, V].
int copy_logits(tt_ctx *ctx, tt_model *md, tt_kvcache *kc, int B, void *logits_out) {
  if (!logits_out) return TT_OK;
  const tt_model_cfg &c = md->cfg;
  const size_t es = esize(c.mode);
  hipError_t e = hipMemcpy2DAsync(logits_out, (size_t)c.V * es, kc->logits, (size_t)md->ld * es,
                                  (size_t)c.V * es, B, hipMemcpyDeviceToDevice, ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "decode: logits copy: %s", hipGetErrorString(e));
  return TT_OK;
}

// One decode step on the cache's device-side position and tokens: embedding,
// every block on B rows with attention over the cache, final LayerNorm,
// logits and the greedy choice into kc->next_dev.  Only kernel launches with
// fixed arguments for a given B (capturable).
int decode_body(tt_ctx *ctx, tt_model *md, tt_kvcache *kc, int B, int pos_hint) {
  const tt_model_cfg &c = md->cfg;
  const tt_mode mode = c.mode;
  const bool lp = tt_lowp(mode);
  const int C = c.C, F = c.F;
  const int S = tt_decode_splits(B, c.NH);
  TT_TRY(tt_embed_decode(ctx, B, C, c.V, kc->tok_dev, kc->pos_dev, md->w + md->off[P_WTE],
                         md->w + md->off[P_WPE], kc->x));
  tt_block_w w;
  LayerWT wt;
  tt_block_g gr;
  for (int l = 0; l < c.L; ++l) {
    layer_views(md, l, w, wt, gr);
    TT_TRY(tt_layernorm_fwd_impl(ctx, mode, B, C, c.ln_eps, kc->x, w.ln1_g, w.ln1_b, kc->ln,
                                 kc->mean, kc->rstd));
    TT_TRY(linear_fwd_gemm(ctx, mode, B, C, 3 * C, kc->ln, C, w.w_qkv, wt.w_qkv, w.b_qkv,
                           EPI_STORE, kc->qkv, 3 * C, lp, nullptr, 0, nullptr, 0));
    TT_TRY(tt_attn_decode(ctx, mode, B, c.NH, kc->pos_dev, pos_hint, c.T_max, kc->qkv, kc->kv[l],
                          kc->att, kc->part, S));
    TT_TRY(linear_fwd_gemm(ctx, mode, B, C, C, kc->att, C, w.w_proj, wt.w_proj, w.b_proj,
                           EPI_RESID, kc->x1, C, false, kc->x, C, nullptr, 0));
    TT_TRY(tt_layernorm_fwd_impl(ctx, mode, B, C, c.ln_eps, kc->x1, w.ln2_g, w.ln2_b, kc->ln,
                                 kc->mean, kc->rstd));
    TT_TRY(linear_fwd_gemm(ctx, mode, B, C, F, kc->ln, C, w.w_fc, wt.w_fc, w.b_fc, EPI_GELU,
                           kc->g, F, lp, nullptr, 0, kc->h, F));
    TT_TRY(linear_fwd_gemm(ctx, mode, B, F, C, kc->g, F, w.w_fcp, wt.w_fcp, w.b_fcp, EPI_RESID,
                           kc->x, C, false, kc->x1, C, nullptr, 0));
  }
  const int lf = p_lnf_g(md);
  TT_TRY(tt_layernorm_fwd_impl(ctx, mode, B, C, c.ln_eps, kc->x, md->w + md->off[lf],
                               md->w + md->off[lf + 1], kc->ln, kc->mean, kc->rstd));
  return logits_and_choice(ctx, md, kc, B, kc->ln, C, kc->next_dev);
}

// Capture decode_body for B sequences into kc->graph (on the cache's own
// stream: the context's stream may be the null stream, which cannot be
// captured).  The graph holds kernel launches only.
int capture_decode(tt_ctx *ctx, tt_model *md, tt_kvcache *kc, int B) {
  if (kc->graph) {
    (void)hipGraphExecDestroy(kc->graph);
    kc->graph = nullptr;
    kc->graph_B = 0;
  }
  hipError_t e = hipStreamBeginCapture(kc->cap, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "decode capture: %s", hipGetErrorString(e));
  hipStream_t saved = ctx->stream;
  ctx->stream = kc->cap;
  int rc = decode_body(ctx, md, kc, B, 0);
  ctx->stream = saved;
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(kc->cap, &graph);
  if (rc == TT_OK && e != hipSuccess)
    rc = tt_set_error(ctx, TT_EHIP, "decode capture: %s", hipGetErrorString(e));
  if (rc == TT_OK) {
    e = hipGraphInstantiate(&kc->graph, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      kc->graph = nullptr;
      rc = tt_set_error(ctx, TT_EHIP, "decode graph: %s", hipGetErrorString(e));
    }
  }
  if (graph) (void)hipGraphDestroy(graph);
  if (rc == TT_OK) kc->graph_B = B;
  return rc;
}

}  // namespace

extern "C" int tt_model_prefill(tt_ctx *ctx, tt_model *md, tt_kvcache *kc, int B, int T,
                                const int32_t *tok, void *logits, int32_t *next) {
  TT_TRY(check_kv(ctx, md, kc, B, tok, next));
  const tt_model_cfg &c = md->cfg;
  TT_REQUIRE(ctx, T >= 1 && T <= c.T_max, "prefill: T must be in [1, %d]", c.T_max);
  const tt_mode mode = c.mode;
  const int N = B * T, C = c.C;
  TT_TRY(tt_embed_fwd(ctx, B, T, C, c.V, tok, md->w + md->off[P_WTE], md->w + md->off[P_WPE],
                      md->xs[0]));
  tt_block_w w;
  LayerWT wt;
  tt_block_g gr;
  for (int l = 0; l < c.L; ++l) {
    layer_views(md, l, w, wt, gr);
    TT_TRY(layer_fwd(ctx, mode, B, T, C, c.NH, c.F, c.ln_eps, w, wt, md->xs[l], md->xs[l + 1],
                     md->layers[l]));
    TT_TRY(tt_kv_store(ctx, mode, B, T, C, c.T_max, md->layers[l].qkv, kc->kv[l]));
  }
  const int lf = p_lnf_g(md);
  TT_TRY(tt_layernorm_fwd_impl(ctx, mode, N, C, c.ln_eps, md->xs[c.L], md->w + md->off[lf],
                               md->w + md->off[lf + 1], md->lnf, md->meanf, md->rstdf));
  // the last position of every sequence: rows b*T + T-1
  const void *last = (const char *)md->lnf + (size_t)(T - 1) * C * esize(mode);
  TT_TRY(logits_and_choice(ctx, md, kc, B, last, T * C, next));
  return copy_logits(ctx, md, kc, B, logits);
}

extern "C" int tt_model_decode(tt_ctx *ctx, tt_model *md, tt_kvcache *kc, int B, int pos,
                               const int32_t *tok, void *logits, int32_t *next) {
  TT_TRY(check_kv(ctx, md, kc, B, tok, next));
  const tt_model_cfg &c = md->cfg;
  TT_REQUIRE(ctx, pos >= 0 && pos < c.T_max, "decode: pos must be in [0, %d)", c.T_max);
  TT_TRY(tt_decode_prep(ctx, B, pos, tok, kc->tok_dev, kc->pos_dev));
  if (ctx->profiling) {
    // per-kernel timing needs every launch on the context's stream
    TT_TRY(decode_body(ctx, md, kc, B, pos));
  } else {
    if (!kc->graph || kc->graph_B != B) TT_TRY(capture_decode(ctx, md, kc, B));
    hipError_t e = hipGraphLaunch(kc->graph, ctx->stream);
    if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "decode graph launch: %s", hipGetErrorString(e));
  }
  TT_TRY(tt_copy_i32(ctx, B, kc->next_dev, next));
  return copy_logits(ctx, md, kc, B, logits);
}

// ------------------------------------------------------------ gradient clipping

extern "C" int tt_model_clip_grad_norm(tt_ctx *ctx, tt_model *md, float max_norm, float *norm) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "clip_grad_norm: bad model handle");
  TT_REQUIRE(ctx, md->ctx == ctx, "clip_grad_norm: model belongs to another context");
  // every slot: padding slots hold zero gradients and add nothing to the norm
  return tt_clip_grad_norm(ctx, md->g, md->n_slots, max_norm, norm);
}

// ------------------------------------------------------------ checkpoints
// The Forge page (section "safetensors格式的安全性优势") reads and writes
// safetensors: an 8-byte little-endian header length, a JSON header naming
// each tensor's dtype, shape and byte range, then the raw data.  Here a
// checkpoint holds the fp32 master weights under the names of the
// HuggingFace GPT-2 files (wte.weight, h.0.attn.c_attn.weight, ...; the token
// table's V rows, W as [in, out]), the AdamW moments as adam_m.<name> and
// adam_v.<name>, and the step count as adam_step (I64 [1]).

namespace {

struct CkTensor {
  std::string name;
  std::vector<int64_t> shape;
  size_t slot, n;
};

std::vector<CkTensor> ck_tensors(const tt_model *md) {
  const tt_model_cfg &c = md->cfg;
  const int64_t C = c.C, F = c.F;
  std::vector<CkTensor> t;
  auto add = [&](int idx, const std::string &name, std::vector<int64_t> shape) {
    size_t n = 1;
    for (int64_t d : shape) n *= (size_t)d;
    t.push_back({name, shape, md->off[idx], n});
  };
  add(P_WTE, "wte.weight", {c.V, C});
  add(P_WPE, "wpe.weight", {c.T_max, C});
  static const char *ln[PER_LAYER] = {"ln_1.weight", "ln_1.bias", "attn.c_attn.weight",
                                      "attn.c_attn.bias", "attn.c_proj.weight", "attn.c_proj.bias",
                                      "ln_2.weight", "ln_2.bias", "mlp.c_fc.weight", "mlp.c_fc.bias",
                                      "mlp.c_proj.weight", "mlp.c_proj.bias"};
  const std::vector<int64_t> sh[PER_LAYER] = {{C}, {C}, {C, 3 * C}, {3 * C}, {C, C}, {C},
                                              {C}, {C}, {C, F}, {F}, {F, C}, {C}};
  for (int l = 0; l < c.L; ++l)
    for (int i = 0; i < PER_LAYER; ++i)
      add(P_LAYER0 + PER_LAYER * l + i, "h." + std::to_string(l) + "." + ln[i], sh[i]);
  const int lf = p_lnf_g(md);
  add(lf, "ln_f.weight", {C});
  add(lf + 1, "ln_f.bias", {C});
  return t;
}

std::string shape_json(const std::vector<int64_t> &s) {
  std::string o = "[";
  for (size_t i = 0; i < s.size(); ++i) o += (i ? "," : "") + std::to_string(s[i]);
  return o + "]";
}

// A JSON reader for safetensors headers: objects, arrays, strings, integers,
// true/false/null.  Values are kept as the tensor entries need them.
struct JVal {
  enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
  double num = 0;
  std::string str;
  std::vector<JVal> arr;
  std::vector<std::pair<std::string, JVal>> obj;
};

struct JParser {
  const std::string &s;
  size_t i = 0;
  bool ok = true;
  explicit JParser(const std::string &src) : s(src) {}
  void ws() { while (i < s.size() && (s[i] == ' ' || s[i] == '\n' || s[i] == '\r' || s[i] == '\t')) ++i; }
  bool eat(char c) { ws(); if (i < s.size() && s[i] == c) { ++i; return true; } return false; }
  std::string string() {
    std::string o;
    if (!eat('"')) { ok = false; return o; }
    while (i < s.size() && s[i] != '"') {
      if (s[i] == '\\' && i + 1 < s.size()) {
        const char e = s[++i];
        o += e == 'n' ? '\n' : e == 't' ? '\t' : e;
        ++i;
      } else {
        o += s[i++];
      }
    }
    if (i >= s.size()) ok = false;
    ++i;
    return o;
  }
  JVal value(int depth = 0) {
    JVal v;
    ws();
    if (!ok || i >= s.size() || depth > 16) { ok = false; return v; }
    const char c = s[i];
    if (c == '{') {
      v.kind = JVal::OBJ; ++i;
      if (eat('}')) return v;
      do {
        std::string k = string();
        if (!eat(':')) { ok = false; return v; }
        v.obj.emplace_back(k, value(depth + 1));
      } while (ok && eat(','));
      if (!eat('}')) ok = false;
    } else if (c == '[') {
      v.kind = JVal::ARR; ++i;
      if (eat(']')) return v;
      do v.arr.push_back(value(depth + 1)); while (ok && eat(','));
      if (!eat(']')) ok = false;
    } else if (c == '"') {
      v.kind = JVal::STR; v.str = string();
    } else if (s.compare(i, 4, "true") == 0) {
      v.kind = JVal::BOOL; v.num = 1; i += 4;
    } else if (s.compare(i, 5, "false") == 0) {
      v.kind = JVal::BOOL; i += 5;
    } else if (s.compare(i, 4, "null") == 0) {
      i += 4;
    } else {
      size_t j = i;
      while (j < s.size() && (isdigit((unsigned char)s[j]) || s[j] == '-' || s[j] == '+' ||
                              s[j] == '.' || s[j] == 'e' || s[j] == 'E')) ++j;
      if (j == i) { ok = false; return v; }
      v.kind = JVal::NUM; v.num = strtod(s.substr(i, j - i).c_str(), nullptr); i = j;
    }
    return v;
  }
};

struct CkEntry {
  std::string dtype;
  std::vector<int64_t> shape;
  uint64_t begin = 0, end = 0;
};

struct FileCloser {
  FILE *f;
  ~FileCloser() { if (f) fclose(f); }
};

}  // namespace

extern "C" int tt_model_save(tt_ctx *ctx, tt_model *md, const char *path, int64_t step) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "model_save: bad model handle");
  TT_REQUIRE(ctx, md->ctx == ctx && path, "model_save: bad arguments");
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "model_save: %s", hipGetErrorString(e));
  const std::vector<CkTensor> ts = ck_tensors(md);
  struct Out { std::string name; const float *src; size_t n; std::vector<int64_t> shape; };
  std::vector<Out> outs;
  for (const char *kind : {"", "adam_m.", "adam_v."})
    for (const CkTensor &t : ts) {
      const float *base = kind[0] == 0 ? md->w : (kind[5] == 'm' ? md->m : md->v);
      outs.push_back({std::string(kind) + t.name, base + t.slot, t.n, t.shape});
    }
  std::string hdr = "{\"__metadata__\":{\"format\":\"pt\"}";
  uint64_t off = 0;
  for (const Out &o : outs) {
    hdr += ",\"" + o.name + "\":{\"dtype\":\"F32\",\"shape\":" + shape_json(o.shape) +
           ",\"data_offsets\":[" + std::to_string(off) + "," + std::to_string(off + 4 * o.n) + "]}";
    off += 4 * o.n;
  }
  hdr += ",\"adam_step\":{\"dtype\":\"I64\",\"shape\":[1],\"data_offsets\":[" +
         std::to_string(off) + "," + std::to_string(off + 8) + "]}}";
  while (hdr.size() % 8) hdr += ' ';
  FileCloser fc{fopen(path, "wb")};
  if (!fc.f) return tt_set_error(ctx, TT_EINVAL, "model_save: cannot open %s", path);
  const uint64_t hl = hdr.size();   // little-endian host
  bool ok = fwrite(&hl, 8, 1, fc.f) == 1 && fwrite(hdr.data(), 1, hl, fc.f) == hl;
  std::vector<float> buf;
  for (const Out &o : outs) {
    if (!ok) break;
    buf.resize(o.n);
    e = hipMemcpy(buf.data(), o.src, o.n * 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "model_save: %s", hipGetErrorString(e));
    ok = fwrite(buf.data(), 4, o.n, fc.f) == o.n;
  }
  ok = ok && fwrite(&step, 8, 1, fc.f) == 1;
  if (!ok) return tt_set_error(ctx, TT_EINVAL, "model_save: write to %s failed", path);
  return TT_OK;
}

extern "C" int tt_model_load_state(tt_ctx *ctx, tt_model *md, const char *path, int64_t *step) {
  TT_TRY(tt_check_ctx(ctx));
  int rc = check_model(md);
  if (rc != TT_OK) return tt_set_error(ctx, rc, "model_load_state: bad model handle");
  TT_REQUIRE(ctx, md->ctx == ctx && path, "model_load_state: bad arguments");
  FileCloser fc{fopen(path, "rb")};
  if (!fc.f) return tt_set_error(ctx, TT_EINVAL, "model_load_state: cannot open %s", path);
  fseek(fc.f, 0, SEEK_END);
  const long fsize = ftell(fc.f);
  fseek(fc.f, 0, SEEK_SET);
  uint64_t hl = 0;
  if (fsize < 8 || fread(&hl, 8, 1, fc.f) != 1 || hl > (uint64_t)fsize - 8 || hl > (1u << 30))
    return tt_set_error(ctx, TT_EINVAL, "model_load_state: %s is not a safetensors file", path);
  std::string hdr(hl, ' ');
  if (fread(&hdr[0], 1, hl, fc.f) != hl)
    return tt_set_error(ctx, TT_EINVAL, "model_load_state: short header in %s", path);
  JParser jp(hdr);
  const JVal root = jp.value();
  if (!jp.ok || root.kind != JVal::OBJ)
    return tt_set_error(ctx, TT_EINVAL, "model_load_state: bad JSON header in %s", path);
  const uint64_t data0 = 8 + hl, dsize = (uint64_t)fsize - data0;
  std::vector<std::pair<std::string, CkEntry>> entries;
  for (const auto &kv : root.obj) {
    if (kv.first == "__metadata__") continue;
    const JVal &v = kv.second;
    CkEntry ce;
    bool good = v.kind == JVal::OBJ;
    for (const auto &f : v.obj) {
      if (f.first == "dtype" && f.second.kind == JVal::STR) ce.dtype = f.second.str;
      else if (f.first == "shape" && f.second.kind == JVal::ARR)
        for (const JVal &d : f.second.arr) ce.shape.push_back((int64_t)d.num);
      else if (f.first == "data_offsets" && f.second.kind == JVal::ARR && f.second.arr.size() == 2) {
        ce.begin = (uint64_t)f.second.arr[0].num;
        ce.end = (uint64_t)f.second.arr[1].num;
      }
    }
    if (!good || ce.end < ce.begin || ce.end > dsize)
      return tt_set_error(ctx, TT_EINVAL, "model_load_state: bad entry %s", kv.first.c_str());
    entries.emplace_back(kv.first, ce);
  }
  auto find = [&](const std::string &name) -> const CkEntry * {
    for (const auto &e : entries)
      if (e.first == name) return &e.second;
    return nullptr;
  };
  const tt_model_cfg &c = md->cfg;
  std::vector<float> buf;
  auto read_into = [&](const CkEntry &ce, float *dst, size_t n) -> int {
    buf.resize(n);
    if (fseek(fc.f, (long)(data0 + ce.begin), SEEK_SET) != 0 || fread(buf.data(), 4, n, fc.f) != n)
      return tt_set_error(ctx, TT_EINVAL, "model_load_state: short data in %s", path);
    hipError_t e = hipMemcpy(dst, buf.data(), n * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "model_load_state: %s", hipGetErrorString(e));
    return TT_OK;
  };
  // everything runs after the stream's pending work, then the copies
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "model_load_state: %s", hipGetErrorString(e));
  for (const CkTensor &t : ck_tensors(md)) {
    const CkEntry *w = find(t.name);
    if (!w) return tt_set_error(ctx, TT_EINVAL, "model_load_state: %s lacks %s", path, t.name.c_str());
    std::vector<int64_t> want = t.shape;
    size_t n = t.n;
    if (t.name == "wte.weight" && w->shape.size() == 2 && w->shape[0] == c.V_pad) {
      want[0] = c.V_pad;   // a padded table is accepted too
      n = (size_t)c.V_pad * c.C;
    }
    for (const char *kind : {"", "adam_m.", "adam_v."}) {
      const CkEntry *ce = kind[0] ? find(std::string(kind) + t.name) : w;
      float *base = kind[0] == 0 ? md->w : (kind[5] == 'm' ? md->m : md->v);
      float *dst = base + t.slot;
      if (t.name == "wte.weight") {   // pad rows stay zero
        const size_t all = (size_t)c.V_pad * c.C;
        TT_TRY(tt_fill_f32(ctx, dst, all, 0.f));
        e = hipStreamSynchronize(ctx->stream);
        if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "model_load_state: %s", hipGetErrorString(e));
      }
      if (!ce) {
        if (kind[0] == 0) return TT_EINVAL;
        if (t.name != "wte.weight") TT_TRY(tt_fill_f32(ctx, dst, t.n, 0.f));
        continue;   // a weights-only file: the moments start at zero
      }
      if (ce->dtype != "F32" || ce->shape != want || ce->end - ce->begin != 4 * n)
        return tt_set_error(ctx, TT_EINVAL, "model_load_state: %s%s has dtype %s or shape "
                            "other than F32 %s", kind, t.name.c_str(), ce->dtype.c_str(),
                            shape_json(want).c_str());
      TT_TRY(read_into(*ce, dst, n));
    }
  }
  if (step) {
    *step = 0;
    const CkEntry *se = find("adam_step");
    if (se) {
      if (se->dtype != "I64" || se->end - se->begin != 8 ||
          fseek(fc.f, (long)(data0 + se->begin), SEEK_SET) != 0 || fread(step, 8, 1, fc.f) != 1)
        return tt_set_error(ctx, TT_EINVAL, "model_load_state: bad adam_step in %s", path);
    }
  }
  // the bf16 shadow and its transposed copy follow the loaded weights
  if (md->lowp) TT_TRY(tt_cast_f32_bf16(ctx, md->n_slots, md->w, md->lowp, md->cfg.mode == TT_FP16));
  return refresh_transposed(md);
}
