// Internal definitions shared by the libtt HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "tt.h"

// ---------------------------------------------------------------------------
// Context
// ---------------------------------------------------------------------------

#define TT_CTX_MAGIC 0x54544358u    // "TTCX"
#define TT_MODEL_MAGIC 0x54544d44u  // "TTMD"
#define TT_SAVED_MAGIC 0x54545342u  // "TTSB"
#define TT_KV_MAGIC 0x54544b56u     // "TTKV"

// One timed kernel launch (profiling mode): HIP events on the context's
// stream around the launch, tagged with the kernel name and its algorithmic
// work (FLOPs for contractions, HBM bytes for bandwidth-bound kernels).
struct tt_prof_rec {
  const char *name;
  double flops, bytes;
  hipEvent_t e0, e1;
};

struct tt_ctx {
  uint32_t magic;
  int device;
  hipStream_t stream;
  char *arena;
  size_t capacity;
  size_t offset;
  size_t mark;
  bool owns_arena;
  int32_t *dev_flags;  // [0]: range error seen in a kernel (token/target id)
  std::string last_error;
  bool profiling = false;
  std::vector<tt_prof_rec> prof;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
};

// Bracket one kernel launch with profiling events (no-op unless enabled).
struct tt_prof_scope {
  tt_ctx *ctx;
  long idx = -1;
  tt_prof_scope(tt_ctx *c, const char *name, double flops, double bytes);
  ~tt_prof_scope();
};

// Workspace of tt_layernorm_bwd_noalloc: a fixed device array per GPU,
// looked up once per device by tt_noalloc_init (called by tt_ctx_create with
// the device current).
constexpr size_t TT_NOALLOC_SCRATCH_BYTES = (size_t)8 << 20;
int tt_noalloc_init(int device);

// Validate a context handle (magic word catches freed or foreign pointers,
// the debug guard idea of the microcrad page's Value.magic).
int tt_check_ctx(const tt_ctx *ctx);
int tt_set_error(tt_ctx *ctx, int status, const char *fmt, ...);
// Report the result of the last kernel launch(es) on this thread.
int tt_check_launch(tt_ctx *ctx, const char *what);
// Arena scratch that lives until the matching tt_scratch_release.
struct tt_scratch_scope {
  tt_ctx *ctx;
  size_t saved;
  explicit tt_scratch_scope(tt_ctx *c) : ctx(c), saved(c->offset) {}
  ~tt_scratch_scope() { ctx->offset = saved; }
};
int tt_arena_alloc(tt_ctx *ctx, size_t bytes, void **p);

#define TT_REQUIRE(ctx, cond, ...)                                 \
  do {                                                             \
    if (!(cond)) return tt_set_error((ctx), TT_EINVAL, __VA_ARGS__); \
  } while (0)

#define TT_TRY(expr)          \
  do {                        \
    int _rc = (expr);         \
    if (_rc != TT_OK) return _rc; \
  } while (0)

static inline bool tt_aligned16(const void *p) { return (((uintptr_t)p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

typedef uint16_t bf16_t;  // bf16 storage
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32), NaN stays NaN.
typedef float tt_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 tt_b2 __attribute__((ext_vector_type(2)));
// Pack two floats into one dword of two bf16 (lo = a).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  tt_f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, tt_b2));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return (bf16_t)(pack_bf2(f, 0.f) & 0xffffu); }
__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// IEEE binary16 (TT_FP16).  Kernels that move 16-bit tensors as raw bits
// keep bf16_t pointers and take a compile-time F16 flag that selects the
// conversions and the MFMA; element-typed kernels use f16_t.
typedef _Float16 f16_t;
typedef _Float16 tt_h2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  tt_f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, tt_h2));
}
__device__ __forceinline__ float h2f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// 16-bit storage format F16 ? binary16 : bf16.
template <bool F16>
__device__ __forceinline__ uint32_t lp_pack2(float a, float b) {
  if constexpr (F16) return pack_h2(a, b);
  else return pack_bf2(a, b);
}
template <bool F16>
__device__ __forceinline__ uint16_t lp_from(float f) {
  return (uint16_t)(lp_pack2<F16>(f, 0.f) & 0xffffu);
}
template <bool F16>
__device__ __forceinline__ float lp_to(uint16_t h) {
  if constexpr (F16) return h2f(h);
  else return bf2f(h);
}
// low / high half of a packed pair
template <bool F16>
__device__ __forceinline__ float lp_lo(uint32_t u) {
  if constexpr (F16) return h2f((uint16_t)(u & 0xffffu));
  else return __uint_as_float(u << 16);
}
template <bool F16>
__device__ __forceinline__ float lp_hi(uint32_t u) {
  if constexpr (F16) return h2f((uint16_t)(u >> 16));
  else return __uint_as_float(u & 0xffff0000u);
}
// 16x16x32 MFMA on eight 16-bit values per lane (bits in a bf16x8_t).
template <bool F16>
__device__ __forceinline__ f32x4_t lp_mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                 __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
inline bool tt_lowp(int mode) { return mode == TT_BF16 || mode == TT_FP16; }

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t *p, size_t i) { return bf2f(p[i]); }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, float v) { p[i] = f2bf(v); }
};
template <> struct Elem<f16_t> {
  __device__ __forceinline__ static float load(const f16_t *p, size_t i) { return (float)p[i]; }
  __device__ __forceinline__ static void store(f16_t *p, size_t i, float v) { p[i] = (f16_t)v; }
};

// Wave64 reductions, every lane receiving the result.  Inside each 16-lane
// row the partners are exchanged with DPP (quad permutations xor 1 and xor
// 2, then the half-row and row mirrors, which pair the already-reduced
// quads and half-rows); across rows with gfx950's row swaps
// (v_permlane16_swap pairs rows 0/1 and 2/3, v_permlane32_swap the two
// halves).  All of it stays in the VALU: no round trip through the LDS
// crossbar, which a shuffle takes.  Each step adds a value to its partner's
// in both lanes of a pair, so every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float2 rowswap16_f(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 rowswap32_f(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_f<0x141>(v);   // row_half_mirror: quad 0 <-> quad 1 of each 8 lanes
  v += dpp_f<0x140>(v);   // row_mirror: half-rows of each 16 lanes
  float2 r = rowswap16_f(v);
  r = rowswap32_f(r.x + r.y);
  return r.x + r.y;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  float2 r = rowswap16_f(v);
  r = rowswap32_f(fmaxf(r.x, r.y));
  return fmaxf(r.x, r.y);
}

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi)(x + 0.044715 x^3).
// The kernels use the identity 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), so
// gelu(x) = x s with s = 1 / (1 + 2^(-2u log2 e)): one hardware exp2 and one
// hardware reciprocal per element instead of an exp and an IEEE division.
// The derivative is s + x s (1 - s) 2u'(x), u'(x) = sqrt(2/pi)(1 + 3 0.044715
// x^2).  Saturation: for large |x| the exp2 goes to 0 or inf and s to 1 or 0.
#define TT_GELU_K 0.7978845608028654f
#define TT_GELU_A 0.044715f
#define TT_GELU_C0 (-2.302208198144325f)    // -2 K log2(e)
#define TT_GELU_C1 (-0.1029432395800235f)   // -2 K A log2(e)
__device__ __forceinline__ float gelu_sig(float x) {   // s = 1 / (1 + exp(-2u))
  const float w = __builtin_fmaf(x * x, TT_GELU_C1, TT_GELU_C0);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(w * x));
}
__device__ __forceinline__ float gelu_f(float x) { return x * gelu_sig(x); }
__device__ __forceinline__ float gelu_grad_f(float x) {
  const float s = gelu_sig(x);
  const float du2 = __builtin_fmaf(x * x, 6.0f * TT_GELU_K * TT_GELU_A, 2.0f * TT_GELU_K);   // 2u'(x)
  return __builtin_fmaf(x * du2, __builtin_fmaf(-s, s, s), s);
}

// ---------------------------------------------------------------------------
// Internal launchers (defined in the .hip files)
// ---------------------------------------------------------------------------

// Epilogue kinds of the GEMM kernel.
enum GemmEpi {
  EPI_STORE = 0,       // out = acc + bias                  (OutT)
  EPI_RESID = 1,       // out(f32) = resid + acc + bias
  EPI_GELU = 2,        // aux = bf(acc + bias) ; out = gelu(acc + bias)
  EPI_GELU_BWD = 3,    // out = acc * gelu'(aux)            (aux = stored preact)
  EPI_ACCUM = 4,       // out(f32) += acc  (atomic when split-K > 1)
  EPI_STORE_ACC = 5    // out(f32) += acc  (non-atomic, split-K must be 1)
};

// C[m,n] = sum_k A(m,k) B(k,n), row/col strides described by the k-major flags:
//   a_kmajor: A(m,k) = A[m*lda + k]   else A[k*lda + m]
//   b_kmajor: B(k,n) = B[n*ldb + k]   else B[k*ldb + n]
struct GemmArgs {
  const void *A; int lda; bool a_kmajor;
  const void *B; int ldb; bool b_kmajor;
  int M, N, K;
  int epi;
  void *out; int ldo; bool out_bf16;
  const float *bias;           // [N] nullable
  const float *resid; int ldr; // EPI_RESID
  void *aux; int ldx;          // EPI_GELU (written preact) / EPI_GELU_BWD (read preact)
  int split_k;                 // >= 1 (EPI_ACCUM only)
  int n_valid;                 // columns >= n_valid of C are not stored (ragged pad); 0 = N
  float *colsum;               // nullable: colsum[n] += sum over rows of the stored output
  int raster;                  // tile order: 0 auto, 1 m fastest, 2 n fastest
  bool overwrite;              // EPI_ACCUM only: store the product instead of adding it
  bool f16;                    // 16-bit operands / output are binary16 (set by tt_gemm)
};
int tt_gemm(tt_ctx *ctx, tt_mode mode, const GemmArgs &g);

// One product of a grouped launch: out[M, N] (fp32, overwritten) =
// sum over k < K of A[k, m] B[k, n], both operands bf16 with the reduction
// index as their row index (A[k * lda + m], B[k * ldb + n]) -- the shape of
// every weight gradient (Xᵀ · dY).  K is shared by the group and given at run
// time; tiles_m, tiles_n, tile0, vec_out and raster_n are filled in by the
// planner.
struct GemmGroupEntry {
  const void *A; const void *B; float *out;
  int lda, ldb, ldo;
  int M, N;
  int tiles_m, tiles_n, tile0, vec_out, raster_n;
};
struct GemmGroup {
  GemmGroupEntry *table = nullptr;   // device copy of the entries
  uint16_t *map = nullptr;           // device: workgroup -> entry (0xffff: padding)
  int n = 0, tiles = 0, grid = 0;
  double mn2 = 0;                    // sum of 2 M N (FLOPs per unit of K)
  double bytes_k = 0, bytes_out = 0;  // operand bytes per unit of K; output bytes
  bool f16 = false;                  // operands are binary16 (else bf16)
};
// Plan a group (entries are copied; the device tables come from the arena
// and stay valid as long as it does).  Every entry must satisfy the bf16
// kernel's layout rules for K up to k_max.
int tt_gemm_group_plan(tt_ctx *ctx, const GemmGroupEntry *entries, int n, int k_max, GemmGroup *out,
                       bool f16 = false);
// Point a planned group at other operands and outputs (same product shapes);
// uploads the table and waits for the stream.
int tt_gemm_group_update(tt_ctx *ctx, GemmGroup &g, const GemmGroupEntry *entries, int n,
                         int k_max);
// Run every product of the group in one launch with reduction length K;
// accumulate: out += product (else out = product).
int tt_gemm_group_run(tt_ctx *ctx, const GemmGroup &g, int K, bool accumulate = false);
// bf16 operands with 16-byte aligned rows (the fast path; called by tt_gemm).
int tt_gemm_bf16(tt_ctx *ctx, const GemmArgs &g);
bool tt_gemm_bf16_ok(const GemmArgs &g);

int tt_layernorm_fwd_impl(tt_ctx *ctx, tt_mode mode, int N, int C, float eps, const float *x,
                          const float *g, const float *b, void *y, float *mean, float *rstd);
// dx = dres + LayerNorm backward, also written as a bf16 copy when dx_bf16 is
// not NULL (dres may alias dx or be NULL); dg, db and dsum (column sums of dx
// as stored, nullable each) are accumulated (+=).
int tt_layernorm_bwd_impl(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                          const float *mean, const float *rstd, const float *g, const float *dy,
                          const float *dres, float *dx, bf16_t *dx_bf16, float *dg, float *db,
                          float *dsum = nullptr);
// The same with the column-partial workspace given: part holds part_groups
// groups of 3 C floats (tt_layernorm_bwd_groups(N, C) are used; every one of
// them is written before it is read, so the workspace needs no clearing).
int tt_layernorm_bwd_ws(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                        const float *mean, const float *rstd, const float *g, const float *dy,
                        const float *dres, float *dx, bf16_t *dx_bf16, float *dg, float *db,
                        float *dsum, float *part, int part_groups);
// The same in two parts: tt_layernorm_bwd_rows writes dx (and its copy) and
// the per-workgroup column partials of dg, db and dsum into part
// ([tt_layernorm_bwd_groups(N, C)][3][C] floats); the partials are added into
// the outputs later, for several calls at once, by
// tt_layernorm_bwd_reduce_batch (table: device array of n entries, all with
// the same N and C).
struct LnReduceEntry {
  const float *part;
  float *dg, *db, *dsum;   // nullable each
};
int tt_layernorm_bwd_groups(int N, int C);
// Largest tt_layernorm_bwd_groups(n, C) over 1 <= n <= N_max: the size (in
// groups of 3 C floats) of a partial buffer that serves every N up to N_max.
int tt_layernorm_bwd_groups_max(int N_max, int C);
// part holds part_groups groups; more needed is TT_EINVAL, nothing enqueued.
int tt_layernorm_bwd_rows(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                          const float *mean, const float *rstd, const float *g, const float *dy,
                          const float *dres, float *dx, bf16_t *dx_bf16, float *part,
                          int part_groups);
int tt_layernorm_bwd_reduce_batch(tt_ctx *ctx, int N, int C, const LnReduceEntry *table, int n);
// Column sums out[n] += sum_m src[m, n]; fmt: the source's tt_mode (float32,
// bf16 or binary16).
int tt_colsum(tt_ctx *ctx, int fmt, int M, int N, int ld, const void *src, float *out);
int tt_fill_f32(tt_ctx *ctx, float *p, size_t n, float v);
// float32 -> 16-bit (bf16, or binary16 when f16), round to nearest even.
int tt_cast_f32_bf16(tt_ctx *ctx, size_t n, const float *src, bf16_t *dst, bool f16 = false);
// Dynamic loss scaling state (device memory).
struct tt_loss_scale {
  float scale;       // current loss scale
  int32_t good;      // clean steps since the scale last changed
  int32_t overflow;  // this step's gradients held inf / NaN
  int32_t skipped;   // steps dropped so far
};
// g *= 1 / scale over n entries; st->overflow |= any entry non-finite.
int tt_unscale_check(tt_ctx *ctx, float *g, size_t n, tt_loss_scale *st);
// Scale update after a step; *out (nullable, device) = the step's overflow.
int tt_loss_scale_update(tt_ctx *ctx, tt_loss_scale *st, int interval, float growth,
                         float backoff, int32_t *out);
int tt_loss_scale_set(tt_ctx *ctx, tt_loss_scale *st, float scale);
// One 64 x 64 tile range of a batched bf16 transpose (src [rows, cols] ->
// dst [cols, rows]); tile0 is the first workgroup of this matrix, tiles are
// numbered row-major with tiles_c = ceil(cols / 64) per tile row.
// src [rows, cols] -> dst [cols, pad_rows] (dst columns rows .. pad_rows-1
// zero); tiles_c = ceil(cols / 64); tile0 = first workgroup of this entry.
struct tt_tdesc {
  const bf16_t *src;
  bf16_t *dst;
  int rows, cols, pad_rows, tiles_c, tile0;
};
// d_dev: device copy of the descriptor table, ordered by tile0.
int tt_transpose_bf16(tt_ctx *ctx, const tt_tdesc *d_dev, int nd, int total_tiles, double elems);
// A few descriptors passed to the kernel by value.
constexpr int TT_TSET = 4;
struct tt_tdesc_set {
  tt_tdesc d[TT_TSET];
  int n = 0, tiles = 0;
  double elems = 0;
};
int tt_tdesc_set_add(tt_tdesc_set &s, const bf16_t *src, bf16_t *dst, int rows, int cols,
                     int pad_rows);
int tt_transpose_bf16_set(tt_ctx *ctx, const tt_tdesc_set &s);
// Inference (decode.hip): copy a prefill's keys and values (qkv columns
// C..3C of rows b*T + t) into the cache [B_max, T_max, 2C]; attention of one
// new position pos over the cache, appending its key and value first, with
// the keys split over up to max_splits workgroups per (sequence, head) whose
// partials go to part (B * NH * max_splits * 66 floats).
int tt_kv_store(tt_ctx *ctx, tt_mode mode, int B, int T, int C, int T_max, const void *qkv,
                void *kv);
// The position comes from device memory (pos_dev), so that one captured
// decode step serves every position; pos_hint only sizes the timer's work.
constexpr int TT_DECODE_MAX_SPLITS = 16;
int tt_decode_splits(int B, int NH);
int tt_attn_decode(tt_ctx *ctx, tt_mode mode, int B, int NH, const int32_t *pos_dev, int pos_hint,
                   int T_max, const void *qkv, void *kv, void *att, float *part, int S);
// pos_dev = pos, tok_dev[0..B) = tok[0..B) (one small launch).
int tt_decode_prep(tt_ctx *ctx, int B, int pos, const int32_t *tok, int32_t *tok_dev,
                   int32_t *pos_dev);
// x[b] = wte[tok_dev[b]] + wpe[*pos_dev].
int tt_embed_decode(tt_ctx *ctx, int B, int C, int V, const int32_t *tok_dev,
                    const int32_t *pos_dev, const float *wte, const float *wpe, float *x);
int tt_copy_i32(tt_ctx *ctx, int n, const int32_t *src, int32_t *dst);
int tt_attn_fwd_impl(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, const void *qkv,
                     void *out, float *lse);
// dbias (nullable) += column sums of dqkv as stored (the qkv bias gradient).
int tt_attn_bwd_impl(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, const void *qkv,
                     const void *out, const float *lse, const void *dout, void *dqkv,
                     float *scratch_D, float *dbias = nullptr);
// bf16 attention kernels (buffer loads, LDS transpose reads); *_ok says
// whether the tensors fit their 32-bit buffer offsets.
bool tt_attn_bf16_ok(int B, int T, int NH);
// f16: the 16-bit tensors are binary16 (else bf16).
int tt_attn_fwd_bf16(tt_ctx *ctx, int B, int T, int NH, const void *qkv, void *out, float *lse,
                     bool f16 = false);
// dbias (nullable) += the column sums of dqkv as stored (the qkv bias
// gradient, [3C] float32).  Dv: [B, NH, T] scratch.
int tt_attn_bwd_bf16(tt_ctx *ctx, int B, int T, int NH, const void *qkv, const void *out,
                     const float *lse, const void *dout, void *dqkv, float *Dv, bool f16 = false,
                     float *dbias = nullptr);
// In-place CE over logits; per_row_loss [N] scratch; loss = mean.
// grad_scale is multiplied by *scale_dev when that is given (the dynamic
// loss scale, kept on the device).
int tt_ce_impl(tt_ctx *ctx, tt_mode mode, int N, int V, int ld, void *logits,
               const int32_t *targets, float *per_row_loss, float *loss, float grad_scale,
               const float *scale_dev = nullptr);
// w_lowp (nullable) receives the 16-bit copy (binary16 when f16); skip
// (nullable, device): a nonzero value drops the update.
int tt_adamw_flat(tt_ctx *ctx, float *w, const float *g, float *m, float *v, bf16_t *w_lowp,
                  size_t n, float lr, float beta1, float beta2, float eps, float wd, int t,
                  bool f16 = false, const int32_t *skip = nullptr);
int tt_check_finite(tt_ctx *ctx, const float *x, size_t n, int32_t *flag);
