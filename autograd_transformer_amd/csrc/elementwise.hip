// Elementwise / gather / scatter kernels: embeddings, AdamW, SGD, GELU,
// fills and casts.  All bandwidth-bound: 16-byte vector accesses, grid-stride.
#include "tt_internal.h"

namespace {

inline int grid_for(size_t n, int per_thread = 4) {
  size_t blocks = (n + (size_t)256 * per_thread - 1) / ((size_t)256 * per_thread);
  if (blocks > 65535u * 16u) blocks = 65535u * 16u;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

// Token + position embedding (tinytorch page §3 item 6):
//   x0[b,t,:] = wte[tok[b,t],:] + wpe[t,:].
// One wave per token row; out-of-range ids poison the row with NaN and raise
// the context's range flag instead of reading outside the table.
__global__ void __launch_bounds__(256) embed_fwd_kernel(int BT, int T, int C, int V,
                                                        const int32_t *__restrict__ tok,
                                                        const float *__restrict__ wte,
                                                        const float *__restrict__ wpe,
                                                        float *__restrict__ x0, int32_t *flags) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= BT) return;
  const int t = row % T;
  const int id = tok[row];
  const bool ok = id >= 0 && id < V;
  if (!ok && lane == 0) atomicOr(flags, 1);
  const float4 *w = (const float4 *)(wte + (size_t)(ok ? id : 0) * C);
  const float4 *p = (const float4 *)(wpe + (size_t)t * C);
  float4 *o = (float4 *)(x0 + (size_t)row * C);
  for (int c = lane; c < C / 4; c += 64) {
    float4 a = w[c], b = p[c];
    o[c] = ok ? make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w)
              : make_float4(NAN, NAN, NAN, NAN);
  }
}

// dwte[tok] += dx0 rows (float atomics: ids repeat, order is not fixed);
// dwpe[t] += sum over the batch (one thread per (t, c), deterministic).
__global__ void __launch_bounds__(256) embed_bwd_tok_kernel(int BT, int C, int V,
                                                            const int32_t *__restrict__ tok,
                                                            const float *__restrict__ dx0,
                                                            float *__restrict__ dwte) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= BT) return;
  const int id = tok[row];
  if (id < 0 || id >= V) return;
  const float *src = dx0 + (size_t)row * C;
  float *dst = dwte + (size_t)id * C;
  for (int c = lane; c < C; c += 64) unsafeAtomicAdd(&dst[c], src[c]);
}

__global__ void __launch_bounds__(256) embed_bwd_pos_kernel(int B, int T, int C,
                                                            const float *__restrict__ dx0,
                                                            float *__restrict__ dwpe) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)T * C) return;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += dx0[(size_t)b * T * C + i];
  dwpe[i] += s;
}

// AdamW on a flat range (tinytorch page §3 item 7; Forge page "核心组件清单").
// bc1 = 1 - beta1^t, bc2 = 1 - beta2^t computed on the host.
__device__ __forceinline__ void adamw_one(float &w, float g, float &m, float &v, float lr,
                                          float b1, float b2, float eps, float wd, float rbc1,
                                          float rbc2) {
  m = b1 * m + (1.0f - b1) * g;
  v = b2 * v + (1.0f - b2) * g * g;
  const float mh = m * rbc1, vh = v * rbc2;
  w = w - lr * (mh / (sqrtf(vh) + eps) + wd * w);
}

// skip (nullable, device): when nonzero the step is dropped (a loss-scaled
// step whose gradients overflowed) -- every thread reads it and returns.
template <bool F16>
__global__ void __launch_bounds__(256) adamw_kernel(size_t n, float *__restrict__ w,
                                                    const float *__restrict__ g,
                                                    float *__restrict__ m, float *__restrict__ v,
                                                    bf16_t *__restrict__ wl, float lr, float b1,
                                                    float b2, float eps, float wd, float rbc1,
                                                    float rbc2, const int32_t *__restrict__ skip) {
  if (skip && *skip) return;
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    // Every byte is touched once: non-temporal (streaming) loads and stores
    // keep the 30 bytes per parameter from displacing cached data (measured
    // 0.697 -> 0.683 ms per 124M-parameter update).
    typedef float v4f __attribute__((ext_vector_type(4)));
    const v4f w_ = __builtin_nontemporal_load((const v4f *)w + i), g_ = __builtin_nontemporal_load((const v4f *)g + i);
    const v4f m_ = __builtin_nontemporal_load((const v4f *)m + i), v_ = __builtin_nontemporal_load((const v4f *)v + i);
    float4 W = make_float4(w_[0], w_[1], w_[2], w_[3]), G = make_float4(g_[0], g_[1], g_[2], g_[3]);
    float4 Mv = make_float4(m_[0], m_[1], m_[2], m_[3]), Vv = make_float4(v_[0], v_[1], v_[2], v_[3]);
    adamw_one(W.x, G.x, Mv.x, Vv.x, lr, b1, b2, eps, wd, rbc1, rbc2);
    adamw_one(W.y, G.y, Mv.y, Vv.y, lr, b1, b2, eps, wd, rbc1, rbc2);
    adamw_one(W.z, G.z, Mv.z, Vv.z, lr, b1, b2, eps, wd, rbc1, rbc2);
    adamw_one(W.w, G.w, Mv.w, Vv.w, lr, b1, b2, eps, wd, rbc1, rbc2);
    __builtin_nontemporal_store((v4f){W.x, W.y, W.z, W.w}, (v4f *)w + i);
    __builtin_nontemporal_store((v4f){Mv.x, Mv.y, Mv.z, Mv.w}, (v4f *)m + i);
    __builtin_nontemporal_store((v4f){Vv.x, Vv.y, Vv.z, Vv.w}, (v4f *)v + i);
    typedef unsigned v2u __attribute__((ext_vector_type(2)));
    if (wl) __builtin_nontemporal_store((v2u){lp_pack2<F16>(W.x, W.y), lp_pack2<F16>(W.z, W.w)}, (v2u *)wl + i);
  }
  // tail
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    float W = w[i], Mv = m[i], Vv = v[i];
    adamw_one(W, g[i], Mv, Vv, lr, b1, b2, eps, wd, rbc1, rbc2);
    w[i] = W; m[i] = Mv; v[i] = Vv;
    if (wl) wl[i] = lp_from<F16>(W);
  }
}

__global__ void __launch_bounds__(256) sgd_kernel(size_t n, float *__restrict__ w,
                                                  const float *__restrict__ g, float lr) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) w[i] -= lr * g[i];
}

__global__ void __launch_bounds__(256) fill_kernel(size_t n, float *__restrict__ p, float val) {
  const size_t n4 = n / 4;
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
    ((float4 *)p)[i] = make_float4(val, val, val, val);
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) p[i] = val;
}

template <bool F16>
__global__ void __launch_bounds__(256) cast_kernel(size_t n, const float *__restrict__ s,
                                                   bf16_t *__restrict__ d) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    d[i] = lp_from<F16>(s[i]);
}

// Dynamic loss scaling (the C++/CUDA page, section 3.4).  The backward of a
// scaled step leaves scale * gradient in g: divide it out and raise the
// overflow flag if any entry is inf or NaN.
__global__ void __launch_bounds__(256) unscale_check_kernel(size_t n, float *__restrict__ g,
                                                            tt_loss_scale *__restrict__ st) {
  const float r = 1.0f / st->scale;
  const size_t n4 = n / 4, stride = (size_t)gridDim.x * 256;
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    float4 v = ((float4 *)g)[i];
    bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
    v.x *= r; v.y *= r; v.z *= r; v.w *= r;
    ((float4 *)g)[i] = v;
  }
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    bad |= !isfinite(g[i]);
    g[i] *= r;
  }
  if (bad) atomicOr(&st->overflow, 1);
}

// After the (possibly skipped) update: halve the scale on overflow and
// restart the clean-step count, else count the step and grow the scale by
// `growth` once `interval` clean steps have passed; report the step's
// overflow flag (nullable out) and clear it for the next step.
__global__ void ls_update_kernel(tt_loss_scale *st, int interval, float growth, float backoff,
                                 int32_t *out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int32_t ov = st->overflow;
  if (ov) {
    st->scale *= backoff;
    st->good = 0;
    st->skipped += 1;
  } else if (++st->good >= interval) {
    st->scale *= growth;
    st->good = 0;
  }
  if (out) *out = ov;
  st->overflow = 0;
}

__global__ void ls_set_kernel(tt_loss_scale *st, float scale) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  st->scale = scale;
  st->good = 0;
  st->overflow = 0;
  st->skipped = 0;
}

// Batched bf16 transpose: descriptor i maps src [rows, cols] (row pitch cols)
// to dst [cols, pad_rows] (row pitch pad_rows >= rows; the columns rows ..
// pad_rows-1 of dst are written as zeros).  One workgroup per 64 x 64 tile,
// staged through LDS so that both the reads and the writes are 16-byte
// coalesced; ragged edges fall back to element accesses.
__device__ __forceinline__ void transpose_tile(const tt_tdesc &d, int local) {
  __shared__ bf16_t t[64][66];
  const int tid = threadIdx.x;
  const bf16_t *src = d.src;
  bf16_t *dst = d.dst;
  const int rows = d.rows, cols = d.cols, prow = d.pad_rows;
  const int r0 = (local / d.tiles_c) * 64, c0 = (local % d.tiles_c) * 64;
  const bool vec_in = (cols & 7) == 0, vec_out = (prow & 7) == 0;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + k * 256;
    const int r = q >> 3, c = (q & 7) * 8;
    const int gr = r0 + r, gc = c0 + c;
    if (gr >= prow) continue;
    if (gr >= rows) {   // padding rows of the source read as zero
      for (int j = 0; j < 8; ++j) t[r][c + j] = 0;
    } else if (vec_in && gc + 7 < cols) {
      const uint4 u = *(const uint4 *)(src + (size_t)gr * cols + gc);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) *(uint32_t *)&t[r][c + 2 * j] = w[j];
    } else {
      for (int j = 0; j < 8; ++j)
        if (gc + j < cols) t[r][c + j] = src[(size_t)gr * cols + gc + j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = tid + k * 256;
    const int c = q >> 3, r = (q & 7) * 8;
    const int gc = c0 + c, gr = r0 + r;
    if (gc >= cols) continue;
    if (vec_out && gr + 7 < prow) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)t[r + 2 * j][c] | ((uint32_t)t[r + 2 * j + 1][c] << 16);
      *(uint4 *)(dst + (size_t)gc * prow + gr) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      for (int j = 0; j < 8; ++j)
        if (gr + j < prow) dst[(size_t)gc * prow + gr + j] = t[r + j][c];
    }
  }
}

// Descriptors in device memory, ordered by tile0 (the model's shadows).
__global__ void __launch_bounds__(256) transpose_bf16_kernel(const tt_tdesc *__restrict__ d,
                                                             int nd) {
  const int b = blockIdx.x;
  int i = 0;
  while (i + 1 < nd && d[i + 1].tile0 <= b) ++i;
  transpose_tile(d[i], b - d[i].tile0);
}

// Up to TT_TSET descriptors passed by value (no device table to upload).
__global__ void __launch_bounds__(256) transpose_bf16_set_kernel(tt_tdesc_set s) {
  const int b = blockIdx.x;
  int i = 0;
#pragma unroll
  for (int j = 1; j < TT_TSET; ++j)
    if (j < s.n && s.d[j].tile0 <= b) i = j;
  tt_tdesc d = s.d[0];
#pragma unroll
  for (int j = 1; j < TT_TSET; ++j)
    if (i == j) d = s.d[j];
  transpose_tile(d, b - d.tile0);
}

template <typename T>
__global__ void __launch_bounds__(256) gelu_fwd_kernel(size_t n, const T *__restrict__ x,
                                                       T *__restrict__ y) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    Elem<T>::store(y, i, gelu_f(Elem<T>::load(x, i)));
}

template <typename T>
__global__ void __launch_bounds__(256) gelu_bwd_kernel(size_t n, const T *__restrict__ x,
                                                       const T *__restrict__ dy,
                                                       T *__restrict__ dx) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    Elem<T>::store(dx, i, Elem<T>::load(dy, i) * gelu_grad_f(Elem<T>::load(x, i)));
}

// flag |= 1 when any of x[0..n) is inf or NaN (x 16-byte aligned: four per
// load; every byte is read once, so the loads are non-temporal).
__global__ void __launch_bounds__(256) finite_kernel(size_t n, const float *__restrict__ x,
                                                     int32_t *__restrict__ flag) {
  const size_t stride = (size_t)gridDim.x * 256;
  const size_t n4 = n / 4;
  bool bad = false;
  typedef float v4f __attribute__((ext_vector_type(4)));
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const v4f v = __builtin_nontemporal_load((const v4f *)x + i);
    bad |= !(isfinite(v[0]) && isfinite(v[1]) && isfinite(v[2]) && isfinite(v[3]));
  }
  for (size_t i = n4 * 4 + (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    bad |= !isfinite(x[i]);
  if (bad) atomicOr(flag, 1);
}

// Global-norm gradient clipping (the C++/CUDA page, section 3.2, clips the
// separately stored gradients by their norm; coefficient max_norm / (norm +
// 1e-6), applied when below 1 -- PyTorch's clip_grad_norm_).  Pass 1: each
// workgroup's sum of squares in float64; pass 2: every workgroup adds the
// CLIP_G partials in the same order (so all agree on the norm bit for bit)
// and scales its share of the gradient.
constexpr int CLIP_G = 1024;

__global__ void __launch_bounds__(256) sumsq_kernel(size_t n, const float *__restrict__ g,
                                                    double *__restrict__ part) {
  double s = 0.0;
  const size_t n4 = n / 4, stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    const float4 v = ((const float4 *)g)[i];
    s += (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
  }
  if (blockIdx.x == 0)
    for (size_t i = n4 * 4 + threadIdx.x; i < n; i += 256) s += (double)g[i] * g[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __shared__ double red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ void __launch_bounds__(256) clip_scale_kernel(size_t n, float *__restrict__ g,
                                                         const double *__restrict__ part,
                                                         float max_norm, float *__restrict__ norm_out) {
  static_assert(CLIP_G == 4 * 256, "four partials per thread");
  __shared__ double red[4];
  __shared__ double coef_s;
  double t = (part[threadIdx.x] + part[threadIdx.x + 256]) +
             (part[threadIdx.x + 512] + part[threadIdx.x + 768]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double nrm = sqrt((red[0] + red[1]) + (red[2] + red[3]));
    coef_s = (double)max_norm / (nrm + 1e-6);
    if (blockIdx.x == 0 && norm_out) *norm_out = (float)nrm;
  }
  __syncthreads();
  const double c = coef_s;
  if (c >= 1.0) return;
  const float cf = (float)c;
  const size_t n4 = n / 4, stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
    float4 v = ((float4 *)g)[i];
    v.x *= cf; v.y *= cf; v.z *= cf; v.w *= cf;
    ((float4 *)g)[i] = v;
  }
  if (blockIdx.x == 0)
    for (size_t i = n4 * 4 + threadIdx.x; i < n; i += 256) g[i] *= cf;
}

}  // namespace

int tt_fill_f32(tt_ctx *ctx, float *p, size_t n, float v) {
  if (n == 0) return TT_OK;
  tt_prof_scope prof(ctx, "fill_kernel", 0.0, 4.0 * n);
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n, 16)), dim3(256), 0, ctx->stream, n, p, v);
  return tt_check_launch(ctx, "fill");
}

int tt_cast_f32_bf16(tt_ctx *ctx, size_t n, const float *src, bf16_t *dst, bool f16) {
  if (n == 0) return TT_OK;
  tt_prof_scope prof(ctx, "cast_kernel", 0.0, 6.0 * n);
  if (f16)
    hipLaunchKernelGGL(cast_kernel<true>, dim3(grid_for(n, 8)), dim3(256), 0, ctx->stream, n, src,
                       dst);
  else
    hipLaunchKernelGGL(cast_kernel<false>, dim3(grid_for(n, 8)), dim3(256), 0, ctx->stream, n, src,
                       dst);
  return tt_check_launch(ctx, "cast");
}

int tt_unscale_check(tt_ctx *ctx, float *g, size_t n, tt_loss_scale *st) {
  if (n == 0) return TT_OK;
  tt_prof_scope prof(ctx, "unscale_check_kernel", 0.0, 8.0 * n);
  hipLaunchKernelGGL(unscale_check_kernel, dim3(grid_for(n, 16)), dim3(256), 0, ctx->stream, n, g,
                     st);
  return tt_check_launch(ctx, "unscale_check");
}

int tt_loss_scale_update(tt_ctx *ctx, tt_loss_scale *st, int interval, float growth,
                         float backoff, int32_t *out) {
  hipLaunchKernelGGL(ls_update_kernel, dim3(1), dim3(64), 0, ctx->stream, st, interval, growth,
                     backoff, out);
  return tt_check_launch(ctx, "loss_scale_update");
}

int tt_loss_scale_set(tt_ctx *ctx, tt_loss_scale *st, float scale) {
  hipLaunchKernelGGL(ls_set_kernel, dim3(1), dim3(64), 0, ctx->stream, st, scale);
  return tt_check_launch(ctx, "loss_scale_set");
}

int tt_transpose_bf16(tt_ctx *ctx, const tt_tdesc *d_dev, int nd, int total_tiles,
                      double elems) {
  if (nd == 0 || total_tiles == 0) return TT_OK;
  tt_prof_scope prof(ctx, "transpose_bf16_kernel", 0.0, 4.0 * elems);
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(total_tiles), dim3(256), 0, ctx->stream, d_dev,
                     nd);
  return tt_check_launch(ctx, "transpose_bf16");
}

int tt_tdesc_set_add(tt_tdesc_set &s, const bf16_t *src, bf16_t *dst, int rows, int cols,
                     int pad_rows) {
  if (s.n >= TT_TSET || rows <= 0 || cols <= 0 || pad_rows < rows) return TT_EINVAL;
  tt_tdesc &d = s.d[s.n++];
  d.src = src; d.dst = dst;
  d.rows = rows; d.cols = cols; d.pad_rows = pad_rows;
  d.tiles_c = (cols + 63) / 64;
  d.tile0 = s.tiles;
  s.tiles += ((pad_rows + 63) / 64) * d.tiles_c;
  s.elems += (double)pad_rows * cols;
  return TT_OK;
}

int tt_transpose_bf16_set(tt_ctx *ctx, const tt_tdesc_set &s) {
  if (s.n == 0 || s.tiles == 0) return TT_OK;
  tt_prof_scope prof(ctx, "transpose_bf16_set_kernel", 0.0, 4.0 * s.elems);
  hipLaunchKernelGGL(transpose_bf16_set_kernel, dim3(s.tiles), dim3(256), 0, ctx->stream, s);
  return tt_check_launch(ctx, "transpose_bf16_set");
}

int tt_adamw_flat(tt_ctx *ctx, float *w, const float *g, float *m, float *v, bf16_t *w_lowp,
                  size_t n, float lr, float beta1, float beta2, float eps, float wd, int t,
                  bool f16, const int32_t *skip) {
  if (n == 0) return TT_OK;
  const float rbc1 = (float)(1.0 / (1.0 - pow((double)beta1, (double)t)));
  const float rbc2 = (float)(1.0 / (1.0 - pow((double)beta2, (double)t)));
  // w, g, m, v read; w, m, v written; optional bf16 copy: 28 (30) bytes per parameter
  tt_prof_scope prof(ctx, "adamw_kernel", 0.0, (28.0 + (w_lowp ? 2.0 : 0.0)) * n);
  if (f16)
    hipLaunchKernelGGL(adamw_kernel<true>, dim3(grid_for(n, 16)), dim3(256), 0, ctx->stream, n, w,
                       g, m, v, w_lowp, lr, beta1, beta2, eps, wd, rbc1, rbc2, skip);
  else
    hipLaunchKernelGGL(adamw_kernel<false>, dim3(grid_for(n, 16)), dim3(256), 0, ctx->stream, n, w,
                       g, m, v, w_lowp, lr, beta1, beta2, eps, wd, rbc1, rbc2, skip);
  return tt_check_launch(ctx, "adamw");
}

int tt_check_finite(tt_ctx *ctx, const float *x, size_t n, int32_t *flag) {
  if (n == 0) return TT_OK;
  TT_REQUIRE(ctx, tt_aligned16(x), "check_finite: x must be 16-byte aligned");
  tt_prof_scope prof(ctx, "finite_kernel", 0.0, 4.0 * n);
  hipLaunchKernelGGL(finite_kernel, dim3(grid_for(n, 16)), dim3(256), 0, ctx->stream, n, x, flag);
  return tt_check_launch(ctx, "finite");
}

extern "C" int tt_embed_fwd(tt_ctx *ctx, int B, int T, int C, int V, const int32_t *tok,
                            const float *wte, const float *wpe, float *x0) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, B >= 0 && T >= 0 && C > 0 && C % 4 == 0 && V > 0, "embed_fwd: bad shape");
  TT_REQUIRE(ctx, tok && wte && wpe && x0, "embed_fwd: NULL pointer");
  TT_REQUIRE(ctx, tt_aligned16(wte) && tt_aligned16(wpe) && tt_aligned16(x0), "embed_fwd: alignment");
  const int BT = B * T;
  if (BT == 0) return TT_OK;
  tt_prof_scope prof(ctx, "embed_fwd_kernel", 0.0, 12.0 * BT * (double)C + 4.0 * BT);
  hipLaunchKernelGGL(embed_fwd_kernel, dim3((BT + 3) / 4), dim3(256), 0, ctx->stream, BT, T, C, V,
                     tok, wte, wpe, x0, ctx->dev_flags);
  return tt_check_launch(ctx, "embed_fwd");
}

extern "C" int tt_embed_bwd(tt_ctx *ctx, int B, int T, int C, int V, const int32_t *tok,
                            const float *dx0, float *dwte, float *dwpe) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, B >= 0 && T >= 0 && C > 0 && V > 0, "embed_bwd: bad shape");
  TT_REQUIRE(ctx, tok && dx0, "embed_bwd: NULL pointer");
  const int BT = B * T;
  if (BT == 0) return TT_OK;
  if (dwte) {
    tt_prof_scope prof(ctx, "embed_bwd_tok_kernel", 0.0, 12.0 * BT * (double)C + 4.0 * BT);
    hipLaunchKernelGGL(embed_bwd_tok_kernel, dim3((BT + 3) / 4), dim3(256), 0, ctx->stream, BT, C, V,
                       tok, dx0, dwte);
    TT_TRY(tt_check_launch(ctx, "embed_bwd_tok"));
  }
  if (dwpe) {
    size_t n = (size_t)T * C;
    tt_prof_scope prof(ctx, "embed_bwd_pos_kernel", 0.0, 4.0 * BT * (double)C + 8.0 * n);
    hipLaunchKernelGGL(embed_bwd_pos_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       ctx->stream, B, T, C, dx0, dwpe);
    TT_TRY(tt_check_launch(ctx, "embed_bwd_pos"));
  }
  return TT_OK;
}

extern "C" int tt_adamw_step(tt_ctx *ctx, const tt_param *params, int count, float lr,
                             float beta1, float beta2, float eps, float wd, int t) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, params != nullptr && count >= 0, "adamw: bad table");
  TT_REQUIRE(ctx, t >= 1, "adamw: t is 1-based");
  for (int i = 0; i < count; ++i) {
    const tt_param &p = params[i];
    TT_REQUIRE(ctx, p.w && p.g && p.m && p.v, "adamw: NULL tensor %d", i);
    TT_REQUIRE(ctx, tt_aligned16(p.w) && tt_aligned16(p.g) && tt_aligned16(p.m) &&
                        tt_aligned16(p.v) && (!p.w_lowp || (((uintptr_t)p.w_lowp) & 7) == 0),
               "adamw: tensor %d misaligned", i);
  }
  for (int i = 0; i < count; ++i) {
    const tt_param &p = params[i];
    TT_TRY(tt_adamw_flat(ctx, p.w, p.g, p.m, p.v, (bf16_t *)p.w_lowp, p.n, lr, beta1, beta2, eps,
                         wd * p.wd_mult, t));
  }
  return TT_OK;
}

extern "C" int tt_sgd_step(tt_ctx *ctx, float *w, const float *g, size_t n, float lr) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, w && g, "sgd: NULL pointer");
  if (n == 0) return TT_OK;
  tt_prof_scope prof(ctx, "sgd_kernel", 0.0, 12.0 * n);
  hipLaunchKernelGGL(sgd_kernel, dim3(grid_for(n)), dim3(256), 0, ctx->stream, n, w, g, lr);
  return tt_check_launch(ctx, "sgd");
}

extern "C" int tt_cast_bf16(tt_ctx *ctx, size_t n, const float *src, void *dst) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, src && dst, "cast: NULL pointer");
  return tt_cast_f32_bf16(ctx, n, src, (bf16_t *)dst);
}

extern "C" int tt_gelu_fwd(tt_ctx *ctx, tt_mode mode, size_t n, const void *x, void *y) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, x && y, "gelu_fwd: NULL pointer");
  if (n == 0) return TT_OK;
  if (mode == TT_BF16)
    hipLaunchKernelGGL(gelu_fwd_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, ctx->stream, n,
                       (const bf16_t *)x, (bf16_t *)y);
  else if (mode == TT_FP16)
    hipLaunchKernelGGL(gelu_fwd_kernel<f16_t>, dim3(grid_for(n)), dim3(256), 0, ctx->stream, n,
                       (const f16_t *)x, (f16_t *)y);
  else
    hipLaunchKernelGGL(gelu_fwd_kernel<float>, dim3(grid_for(n)), dim3(256), 0, ctx->stream, n,
                       (const float *)x, (float *)y);
  return tt_check_launch(ctx, "gelu_fwd");
}

extern "C" int tt_gelu_bwd(tt_ctx *ctx, tt_mode mode, size_t n, const void *x, const void *dy,
                           void *dx) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, x && dy && dx, "gelu_bwd: NULL pointer");
  if (n == 0) return TT_OK;
  if (mode == TT_BF16)
    hipLaunchKernelGGL(gelu_bwd_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, ctx->stream, n,
                       (const bf16_t *)x, (const bf16_t *)dy, (bf16_t *)dx);
  else if (mode == TT_FP16)
    hipLaunchKernelGGL(gelu_bwd_kernel<f16_t>, dim3(grid_for(n)), dim3(256), 0, ctx->stream, n,
                       (const f16_t *)x, (const f16_t *)dy, (f16_t *)dx);
  else
    hipLaunchKernelGGL(gelu_bwd_kernel<float>, dim3(grid_for(n)), dim3(256), 0, ctx->stream, n,
                       (const float *)x, (const float *)dy, (float *)dx);
  return tt_check_launch(ctx, "gelu_bwd");
}

extern "C" int tt_clip_grad_norm(tt_ctx *ctx, float *g, size_t n, float max_norm, float *norm) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, g && n > 0 && tt_aligned16(g), "clip_grad_norm: bad gradient buffer");
  TT_REQUIRE(ctx, max_norm > 0.f, "clip_grad_norm: max_norm must be positive");
  tt_scratch_scope scope(ctx);
  void *part;
  TT_TRY(tt_arena_alloc(ctx, CLIP_G * sizeof(double), &part));
  {
    tt_prof_scope prof(ctx, "sumsq_kernel", 0.0, 4.0 * n);
    hipLaunchKernelGGL(sumsq_kernel, dim3(CLIP_G), dim3(256), 0, ctx->stream, n, g, (double *)part);
    TT_TRY(tt_check_launch(ctx, "sumsq"));
  }
  tt_prof_scope prof(ctx, "clip_scale_kernel", 0.0, 8.0 * n);
  hipLaunchKernelGGL(clip_scale_kernel, dim3(CLIP_G), dim3(256), 0, ctx->stream, n, g,
                     (const double *)part, max_norm, norm);
  return tt_check_launch(ctx, "clip_scale");
}
