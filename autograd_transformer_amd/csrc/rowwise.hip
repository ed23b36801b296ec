// Bandwidth-bound kernels: LayerNorm forward/backward, fused softmax +
// cross-entropy, column sums (bias gradients).  One wave (64 lanes) owns a
// row; row statistics are wave-shuffle reductions; loads are 16-byte vectors.
#include "tt_internal.h"

namespace {

// LN_MAXV: float4 per lane (template); C <= 64 * 4 * LN_MAXV, at most 4096.

// LayerNorm forward — tinytorch page §4 (subtract the mean, divide by the
// standard deviation, scale by the weight, add the bias); biased variance,
// eps inside the square root.  Two-pass statistics from registers.
template <bool OUT_BF16, int LN_MAXV>
__global__ void __launch_bounds__(256) layernorm_fwd_kernel(int N, int C, float eps,
                                                            const float *__restrict__ x,
                                                            const float *__restrict__ g,
                                                            const float *__restrict__ b,
                                                            void *__restrict__ y,
                                                            float *__restrict__ mean_out,
                                                            float *__restrict__ rstd_out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  const int nv = C >> 2;
  const float4 *xr = (const float4 *)(x + (size_t)row * C);
  float4 v[LN_MAXV];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = lane + i * 64;
    if (c < nv) {
      v[i] = xr[c];
      s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
    }
  }
  const float mean = wave_sum(s) / (float)C;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = lane + i * 64;
    if (c < nv) {
      float a = v[i].x - mean, bb = v[i].y - mean, cc = v[i].z - mean, d = v[i].w - mean;
      q += (a * a + bb * bb) + (cc * cc + d * d);
    }
  }
  const float var = wave_sum(q) / (float)C;
  const float rstd = 1.0f / sqrtf(var + eps);
  const float4 *g4 = (const float4 *)g;
  const float4 *b4 = (const float4 *)b;
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = lane + i * 64;
    if (c < nv) {
      float4 gg = g4[c], bb = b4[c];
      float o0 = (v[i].x - mean) * rstd * gg.x + bb.x;
      float o1 = (v[i].y - mean) * rstd * gg.y + bb.y;
      float o2 = (v[i].z - mean) * rstd * gg.z + bb.z;
      float o3 = (v[i].w - mean) * rstd * gg.w + bb.w;
      if (OUT_BF16) {
        uint2 pk = make_uint2(pack_bf2(o0, o1), pack_bf2(o2, o3));
        ((uint2 *)((bf16_t *)y + (size_t)row * C))[c] = pk;
      } else {
        ((float4 *)((float *)y + (size_t)row * C))[c] = make_float4(o0, o1, o2, o3);
      }
    }
  }
  if (lane == 0) {
    if (mean_out) mean_out[row] = mean;
    if (rstd_out) rstd_out[row] = rstd;
  }
}

// LayerNorm backward: with g_i = dy_i * gamma_i and xhat = (x - mean) * rstd,
//   dx = dres + rstd * (g - mean(g) - xhat * mean(g * xhat));
//   dgamma += sum_rows dy * xhat ; dbeta += sum_rows dy.
// A block of 4 waves handles ROWS_PER_BLOCK rows; gamma/beta partials are
// kept per lane in registers and flushed with one atomic per column.
constexpr int LNB_ROWS = 32;

template <int LN_MAXV>
__global__ void __launch_bounds__(256) layernorm_bwd_kernel(
    int N, int C, const float *__restrict__ x, const float *__restrict__ mean,
    const float *__restrict__ rstd, const float *__restrict__ gamma, const float *__restrict__ dy,
    const float *dres, float *dx, bf16_t *__restrict__ dx_bf16, float *__restrict__ dgamma,
    float *__restrict__ dbeta) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nv = C >> 2;
  const float4 *g4 = (const float4 *)gamma;
  float4 pg[LN_MAXV], pb[LN_MAXV];
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    pg[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    pb[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const int r0 = blockIdx.x * LNB_ROWS;
  for (int rr = wave; rr < LNB_ROWS; rr += 4) {
    const int row = r0 + rr;
    if (row >= N) break;
    const float mu = mean[row], rs = rstd[row];
    const float4 *xr = (const float4 *)(x + (size_t)row * C);
    const float4 *dyr = (const float4 *)(dy + (size_t)row * C);
    float4 xh[LN_MAXV], gg[LN_MAXV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      int c = lane + i * 64;
      if (c < nv) {
        float4 xv = xr[c], d = dyr[c], ga = g4[c];
        xh[i] = make_float4((xv.x - mu) * rs, (xv.y - mu) * rs, (xv.z - mu) * rs, (xv.w - mu) * rs);
        gg[i] = make_float4(d.x * ga.x, d.y * ga.y, d.z * ga.z, d.w * ga.w);
        s1 += (gg[i].x + gg[i].y) + (gg[i].z + gg[i].w);
        s2 += (gg[i].x * xh[i].x + gg[i].y * xh[i].y) + (gg[i].z * xh[i].z + gg[i].w * xh[i].w);
        pg[i].x += d.x * xh[i].x; pg[i].y += d.y * xh[i].y;
        pg[i].z += d.z * xh[i].z; pg[i].w += d.w * xh[i].w;
        pb[i].x += d.x; pb[i].y += d.y; pb[i].z += d.z; pb[i].w += d.w;
      }
    }
    const float m1 = wave_sum(s1) / (float)C;
    const float m2 = wave_sum(s2) / (float)C;
    float4 *dxr = (float4 *)(dx + (size_t)row * C);
    const float4 *drr = dres ? (const float4 *)(dres + (size_t)row * C) : nullptr;
#pragma unroll
    for (int i = 0; i < LN_MAXV; ++i) {
      int c = lane + i * 64;
      if (c < nv) {
        float4 o;
        o.x = rs * (gg[i].x - m1 - xh[i].x * m2);
        o.y = rs * (gg[i].y - m1 - xh[i].y * m2);
        o.z = rs * (gg[i].z - m1 - xh[i].z * m2);
        o.w = rs * (gg[i].w - m1 - xh[i].w * m2);
        if (drr) {
          float4 r = drr[c];
          o.x += r.x; o.y += r.y; o.z += r.z; o.w += r.w;
        }
        dxr[c] = o;
        if (dx_bf16)
          ((uint2 *)(dx_bf16 + (size_t)row * C))[c] =
              make_uint2(pack_bf2(o.x, o.y), pack_bf2(o.z, o.w));
      }
    }
  }
  // Combine the 4 waves' partials through LDS, then one atomic per column.
  __shared__ float red[2][4096];
  for (int i = threadIdx.x; i < C; i += 256) { red[0][i] = 0.f; red[1][i] = 0.f; }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    int c = lane + i * 64;
    if (c < nv) {
      atomicAdd(&red[0][4 * c + 0], pg[i].x); atomicAdd(&red[0][4 * c + 1], pg[i].y);
      atomicAdd(&red[0][4 * c + 2], pg[i].z); atomicAdd(&red[0][4 * c + 3], pg[i].w);
      atomicAdd(&red[1][4 * c + 0], pb[i].x); atomicAdd(&red[1][4 * c + 1], pb[i].y);
      atomicAdd(&red[1][4 * c + 2], pb[i].z); atomicAdd(&red[1][4 * c + 3], pb[i].w);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < C; i += 256) {
    if (dgamma) unsafeAtomicAdd(&dgamma[i], red[0][i]);
    if (dbeta) unsafeAtomicAdd(&dbeta[i], red[1][i]);
  }
}

// Column sums out[n] += sum_m src[m, n] (bias gradients).  Each block sums a
// strip of 64 columns over a slice of rows, then one atomic per column.
template <bool BF16>
__global__ void __launch_bounds__(256) colsum_kernel(int M, int N, int ld, int rows_per_block,
                                                     const void *__restrict__ src,
                                                     float *__restrict__ out) {
  const int col = blockIdx.x * 64 + (threadIdx.x & 63);
  const int part = threadIdx.x >> 6;
  const int m0 = blockIdx.y * rows_per_block;
  const int m1 = min(M, m0 + rows_per_block);
  float s = 0.f;
  if (col < N) {
    for (int m = m0 + part; m < m1; m += 4) {
      s += BF16 ? bf2f(((const bf16_t *)src)[(size_t)m * ld + col])
                : ((const float *)src)[(size_t)m * ld + col];
    }
  }
  __shared__ float red[4][64];
  red[part][threadIdx.x & 63] = s;
  __syncthreads();
  if (part == 0 && col < N) {
    float t = (red[0][threadIdx.x] + red[1][threadIdx.x]) + (red[2][threadIdx.x] + red[3][threadIdx.x]);
    unsafeAtomicAdd(&out[col], t);
  }
}

// Fused softmax + cross-entropy over one row of logits per block (tinytorch
// page §3 item 5; Forge page "瓶颈分析是否合理": fuse the max, exp-sum and
// normalise passes).  Pass 1 keeps a running (max, sum of exp) per thread —
// the online form of the max-subtracted softmax — and merges them; pass 2
// overwrites the row with dz = (exp(z - lse) - [v == y]) * scale and zeroes
// the padding columns.
template <bool BF16>
__global__ void __launch_bounds__(256) ce_kernel(int N, int V, int ld, void *logits,
                                                 const int32_t *__restrict__ targets,
                                                 float *__restrict__ row_loss, float scale,
                                                 int32_t *flags) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int y = targets[row];
  const bool y_ok = (y >= 0 && y < V);
  float m = -INFINITY, s = 0.f;
  if (BF16) {
    const bf16_t *z = (const bf16_t *)logits + (size_t)row * ld;
    // 8 values per 16-byte load; ld % 8 == 0 is required by the host.
    const int nv8 = V >> 3;
    for (int i = tid; i < nv8; i += 256) {
      uint4 u = ((const uint4 *)z)[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(w[q] << 16);
        v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
      float mx = v[0];
#pragma unroll
      for (int q = 1; q < 8; ++q) mx = fmaxf(mx, v[q]);
      float nm = fmaxf(m, mx);
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += __expf(v[q] - nm);
      s = s * __expf(m - nm) + acc;
      m = nm;
    }
    for (int i = (nv8 << 3) + tid; i < V; i += 256) {
      float v = bf2f(z[i]);
      float nm = fmaxf(m, v);
      s = s * __expf(m - nm) + __expf(v - nm);
      m = nm;
    }
  } else {
    const float *z = (const float *)logits + (size_t)row * ld;
    for (int i = tid; i < V; i += 256) {
      float v = z[i];
      float nm = fmaxf(m, v);
      s = s * __expf(m - nm) + __expf(v - nm);
      m = nm;
    }
  }
  // merge (m, s) across the block
  __shared__ float sm[256], ss[256];
  float wm = wave_max(m);
  float ws = wave_sum(m == -INFINITY ? 0.f : s * __expf(m - wm));
  if ((tid & 63) == 0) { sm[tid >> 6] = wm; ss[tid >> 6] = ws; }
  __syncthreads();
  float gm = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
  float gs = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) gs += (sm[w] == -INFINITY) ? 0.f : ss[w] * __expf(sm[w] - gm);
  const float lse = gm + __logf(gs);
  __syncthreads();
  if (tid == 0) {
    float zy;
    if (BF16)
      zy = y_ok ? bf2f(((const bf16_t *)logits)[(size_t)row * ld + y]) : NAN;
    else
      zy = y_ok ? ((const float *)logits)[(size_t)row * ld + y] : NAN;
    row_loss[row] = lse - zy;
    if (!y_ok) atomicOr(flags, 1);
  }
  __syncthreads();  // the target logit is read before it is overwritten
  if (BF16) {
    bf16_t *z = (bf16_t *)logits + (size_t)row * ld;
    const int nv8 = ld >> 3;
    for (int i = tid; i < nv8; i += 256) {
      uint4 u = ((const uint4 *)z)[i];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int c0 = i * 8 + 2 * q, c1 = c0 + 1;
        float v0 = __uint_as_float(w[q] << 16), v1 = __uint_as_float(w[q] & 0xffff0000u);
        float d0 = c0 < V ? (__expf(v0 - lse) - (c0 == y ? 1.f : 0.f)) * scale : 0.f;
        float d1 = c1 < V ? (__expf(v1 - lse) - (c1 == y ? 1.f : 0.f)) * scale : 0.f;
        o[q] = pack_bf2(d0, d1);
      }
      ((uint4 *)z)[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
    float *z = (float *)logits + (size_t)row * ld;
    for (int i = tid; i < ld; i += 256) {
      float d = 0.f;
      if (i < V) d = (__expf(z[i] - lse) - (i == y ? 1.f : 0.f)) * scale;
      z[i] = d;
    }
  }
}

// Deterministic mean of n floats in one block.
__global__ void __launch_bounds__(256) mean_kernel(int n, const float *__restrict__ src,
                                                   float *__restrict__ out) {
  float s = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) s += src[i];
  __shared__ float red[4];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = ((red[0] + red[1]) + (red[2] + red[3])) / (float)n;
}

}  // namespace

int tt_layernorm_fwd_impl(tt_ctx *ctx, tt_mode mode, int N, int C, float eps, const float *x,
                          const float *g, const float *b, void *y, float *mean, float *rstd) {
  TT_REQUIRE(ctx, N >= 0 && C > 0 && C % 4 == 0 && C <= 4096, "layernorm: need C %% 4 == 0, C <= 4096");
  TT_REQUIRE(ctx, x && g && b && y, "layernorm_fwd: NULL pointer");
  if (N == 0) return TT_OK;
  dim3 grid((N + 3) / 4);
  const int nv = (C / 4 + 63) / 64;
  tt_prof_scope prof(ctx, "layernorm_fwd_kernel", 0.0,
                     (double)N * C * (4.0 + (mode == TT_BF16 ? 2.0 : 4.0)) + 8.0 * C + 8.0 * N);
#define TT_LNF(NV)                                                                              \
  if (nv <= NV) {                                                                               \
    if (mode == TT_BF16)                                                                        \
      hipLaunchKernelGGL((layernorm_fwd_kernel<true, NV>), grid, dim3(256), 0, ctx->stream, N, C, \
                         eps, x, g, b, y, mean, rstd);                                          \
    else                                                                                        \
      hipLaunchKernelGGL((layernorm_fwd_kernel<false, NV>), grid, dim3(256), 0, ctx->stream, N,   \
                         C, eps, x, g, b, y, mean, rstd);                                       \
    return tt_check_launch(ctx, "layernorm_fwd");                                               \
  }
  TT_LNF(1) TT_LNF(2) TT_LNF(3) TT_LNF(4) TT_LNF(8) TT_LNF(16)
#undef TT_LNF
  return TT_EUNSUPPORTED;
}

int tt_layernorm_bwd_impl(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                          const float *mean, const float *rstd, const float *g, const float *dy,
                          const float *dres, float *dx, bf16_t *dx_bf16, float *dg, float *db) {
  (void)mode;
  TT_REQUIRE(ctx, N >= 0 && C > 0 && C % 4 == 0 && C <= 4096, "layernorm: need C %% 4 == 0, C <= 4096");
  TT_REQUIRE(ctx, x && mean && rstd && g && dy && dx, "layernorm_bwd: NULL pointer");
  if (N == 0) return TT_OK;
  dim3 grid((N + LNB_ROWS - 1) / LNB_ROWS);
  const int nv = (C / 4 + 63) / 64;
  tt_prof_scope prof(ctx, "layernorm_bwd_kernel", 0.0,
                     (double)N * C * (12.0 + (dres ? 4.0 : 0.0) + (dx_bf16 ? 2.0 : 0.0)) +
                         16.0 * C + 8.0 * N);
#define TT_LNB(NV)                                                                              \
  if (nv <= NV) {                                                                               \
    hipLaunchKernelGGL((layernorm_bwd_kernel<NV>), grid, dim3(256), 0, ctx->stream, N, C, x, mean, \
                       rstd, g, dy, dres, dx, dx_bf16, dg, db);                                 \
    return tt_check_launch(ctx, "layernorm_bwd");                                               \
  }
  TT_LNB(1) TT_LNB(2) TT_LNB(3) TT_LNB(4) TT_LNB(8) TT_LNB(16)
#undef TT_LNB
  return TT_EUNSUPPORTED;
}

int tt_colsum(tt_ctx *ctx, bool src_bf16, int M, int N, int ld, const void *src, float *out) {
  if (M == 0 || N == 0) return TT_OK;
  int colblocks = (N + 63) / 64;
  int rowsplit = 1;
  while (colblocks * rowsplit < 1024 && rowsplit * 64 < M) rowsplit *= 2;
  int rpb = (M + rowsplit - 1) / rowsplit;
  dim3 grid(colblocks, (M + rpb - 1) / rpb);
  tt_prof_scope prof(ctx, "colsum_kernel", 0.0, (double)M * N * (src_bf16 ? 2.0 : 4.0) + 4.0 * N);
  if (src_bf16)
    hipLaunchKernelGGL(colsum_kernel<true>, grid, dim3(256), 0, ctx->stream, M, N, ld, rpb, src, out);
  else
    hipLaunchKernelGGL(colsum_kernel<false>, grid, dim3(256), 0, ctx->stream, M, N, ld, rpb, src, out);
  return tt_check_launch(ctx, "colsum");
}

int tt_ce_impl(tt_ctx *ctx, tt_mode mode, int N, int V, int ld, void *logits,
               const int32_t *targets, float *per_row_loss, float *loss, float grad_scale) {
  TT_REQUIRE(ctx, N > 0 && V > 0 && ld >= V, "ce: bad shape N=%d V=%d ld=%d", N, V, ld);
  TT_REQUIRE(ctx, logits && targets && per_row_loss && loss, "ce: NULL pointer");
  {
  tt_prof_scope prof(ctx, "ce_kernel", 0.0, 2.0 * N * (double)ld * (mode == TT_BF16 ? 2.0 : 4.0) + 8.0 * N);
  if (mode == TT_BF16) {
    TT_REQUIRE(ctx, ld % 8 == 0 && tt_aligned16(logits), "ce(bf16): ld %% 8 and 16-byte alignment required");
    hipLaunchKernelGGL(ce_kernel<true>, dim3(N), dim3(256), 0, ctx->stream, N, V, ld, logits,
                       targets, per_row_loss, grad_scale, ctx->dev_flags);
  } else {
    hipLaunchKernelGGL(ce_kernel<false>, dim3(N), dim3(256), 0, ctx->stream, N, V, ld, logits,
                       targets, per_row_loss, grad_scale, ctx->dev_flags);
  }
  }
  TT_TRY(tt_check_launch(ctx, "ce"));
  tt_prof_scope prof(ctx, "mean_kernel", 0.0, 4.0 * N);
  hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(256), 0, ctx->stream, N, per_row_loss, loss);
  return tt_check_launch(ctx, "ce_mean");
}
