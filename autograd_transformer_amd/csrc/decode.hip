// Inference kernels: the greedy choice of the next token, the key/value cache
// and the attention of one new position over that cache.
//
// The Forge page (sections "性能瓶颈与未来路线图" and "瓶颈分析是否合理")
// names the missing KV cache as its main inference cost and describes it:
// under causal attention the keys and values of earlier positions never
// change, so each step computes q, k, v of the new token only, appends k and
// v to the cache and attends over all of it.  Here the cache lives in HBM,
// [B_max, T_max, 2C] per layer (each position's keys, then its values; head
// h at columns h*64 .. h*64+63), so a new token costs one row of every
// product plus one read of the cache.
#include <limits.h>

#include <algorithm>

#include "tt_internal.h"

namespace {

// Order of the greedy choice: NaN above every number (NumPy's argmax rule),
// then larger values, then lower indices (ties resolve to the first).
__device__ __forceinline__ bool am_better(float b, int ib, float a, int ia) {
  const bool nb = b != b, na = a != a;
  if (nb != na) return nb;
  if (!nb && b != a) return b > a;
  return ib < ia;
}

__device__ __forceinline__ void am_take(float &best, int &bi, float v, int i) {
  if (am_better(v, i, best, bi)) {
    best = v;
    bi = i;
  }
}

// One workgroup per row; each thread scans its columns in increasing order,
// then (value, index) pairs are reduced across the wave and the workgroup.
// VEC: the row is read as 16-byte vectors (aligned rows, ld a multiple of the
// vector width); columns >= V are skipped.
template <bool BF16, bool VEC>
__global__ void __launch_bounds__(256) argmax_kernel(int V, int ld, const void *logits,
                                                     int32_t *__restrict__ out) {
  const int row = blockIdx.x, tid = threadIdx.x;
  float best = -INFINITY;
  int bi = INT_MAX;
  if constexpr (BF16) {
    const bf16_t *z = (const bf16_t *)logits + (size_t)row * ld;
    if constexpr (VEC) {
      for (int c8 = tid; c8 * 8 < V; c8 += 256) {
        const uint4 u = ((const uint4 *)z)[c8];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int i = c8 * 8 + q;
          const float v = __uint_as_float((q & 1) ? (w[q >> 1] & 0xffff0000u) : (w[q >> 1] << 16));
          if (i < V) am_take(best, bi, v, i);
        }
      }
    } else {
      for (int i = tid; i < V; i += 256) am_take(best, bi, bf2f(z[i]), i);
    }
  } else {
    const float *z = (const float *)logits + (size_t)row * ld;
    if constexpr (VEC) {
      for (int c4 = tid; c4 * 4 < V; c4 += 256) {
        const float4 u = ((const float4 *)z)[c4];
        const float w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c4 * 4 + q < V) am_take(best, bi, w[q], c4 * 4 + q);
      }
    } else {
      for (int i = tid; i < V; i += 256) am_take(best, bi, z[i], i);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    am_take(best, bi, ob, oi);
  }
  __shared__ float rb[4];
  __shared__ int ri[4];
  const int wave = tid >> 6;
  if ((tid & 63) == 0) {
    rb[wave] = best;
    ri[wave] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < 4; ++w) am_take(best, bi, rb[w], ri[w]);
    out[row] = bi;
  }
}

// kv[b, t, 0 .. 2C) = qkv[b * T + t, C .. 3C) for t < T: the keys and values
// a prefill computed, into the cache.  One workgroup per position, 16-byte
// copies (2C elements are whole vectors: C is a multiple of 8).
template <typename E>
__global__ void __launch_bounds__(256) kv_store_kernel(int T, int C, int T_max,
                                                       const E *__restrict__ qkv,
                                                       E *__restrict__ kv) {
  const int row = blockIdx.x;
  const int b = row / T, t = row % T;
  const uint4 *src = (const uint4 *)(qkv + (size_t)row * 3 * C + C);
  uint4 *dst = (uint4 *)(kv + ((size_t)b * T_max + t) * 2 * C);
  const int nvec = 2 * C * (int)sizeof(E) / 16;
  for (int i = threadIdx.x; i < nvec; i += 256) dst[i] = src[i];
}

__device__ __forceinline__ float ld_elem(const bf16_t *p, size_t i) { return bf2f(p[i]); }
__device__ __forceinline__ float ld_elem(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ void st_elem(bf16_t *p, size_t i, float v) { p[i] = f2bf(v); }
__device__ __forceinline__ void st_elem(float *p, size_t i, float v) { p[i] = v; }

template <typename E>
__device__ __forceinline__ void load_row64(const E *p, float (&k)[64]) {
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint4 u = ((const uint4 *)p)[v];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        k[v * 8 + 2 * q] = __uint_as_float(w[q] << 16);
        k[v * 8 + 2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float4 u = ((const float4 *)p)[v];
      k[v * 4] = u.x; k[v * 4 + 1] = u.y; k[v * 4 + 2] = u.z; k[v * 4 + 3] = u.w;
    }
  }
}

// Attention of the token at position pos of every sequence: the last row of
// the causal softmax attention (tinytorch page §4; Forge page "最硬的一关"),
// scale 1/8, keys 0..pos.  The keys are split into S ranges so that B*NH*S
// workgroups share the cache read: workgroup (sequence, head, split) writes
// the partial (max m, sum l of exp(score - m), sum o of exp(score - m) v) of
// its range, and attn_decode_combine_kernel merges the S partials (the
// online-softmax rescaling of the training kernels).  The workgroup whose
// range holds pos appends the new key and value to the cache and uses its
// own copy of them; no other workgroup touches row pos.
constexpr int DEC_PART = 66;   // floats per partial: m, l, o[64]

template <typename E>
__global__ void __launch_bounds__(256) attn_decode_kernel(int NH, const int32_t *__restrict__ pos_p,
                                                          int T_max, int S,
                                                          const E *__restrict__ qkv, E *kv,
                                                          float *__restrict__ part_out) {
  extern __shared__ float sc[];   // [chunk] scores, then exp(score - m)
  const int pos = *pos_p;
  __shared__ float q[64], kn[64], vn[64];
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x / S, split = blockIdx.x % S;
  const int b = bh / NH, h = bh % NH;
  const int C = NH * 64;
  const int chunk = (pos + 1 + S - 1) / S;
  const int t0 = split * chunk, t1 = min(pos + 1, t0 + chunk);   // keys [t0, t1)
  float *po = part_out + (size_t)blockIdx.x * DEC_PART;
  const E *row = qkv + (size_t)b * 3 * C + h * 64;
  E *cache = kv + (size_t)b * T_max * 2 * C + h * 64;   // key of position t at t * 2C
  const bool owns_pos = t0 <= pos && pos < t1;
  if (tid < 64) {
    q[tid] = ld_elem(row, tid);
    if (owns_pos) {
      kn[tid] = ld_elem(row + C, tid);
      vn[tid] = ld_elem(row + 2 * C, tid);
      cache[(size_t)pos * 2 * C + tid] = row[C + tid];
      cache[(size_t)pos * 2 * C + C + tid] = row[2 * C + tid];
    }
  }
  if (t0 >= t1) {   // empty range (uniform over the workgroup)
    if (tid < DEC_PART) po[tid] = tid == 0 ? -INFINITY : 0.f;
    return;
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int t = t0 + tid; t < t1; t += 256) {
    float k[64];
    if (t == pos) {
#pragma unroll
      for (int d = 0; d < 64; ++d) k[d] = kn[d];
    } else {
      load_row64(cache + (size_t)t * 2 * C, k);
    }
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < 64; ++d) s += q[d] * k[d];
    s *= 0.125f;
    sc[t - t0] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  float sum = 0.f;
  for (int t = t0 + tid; t < t1; t += 256) {
    const float e = __expf(sc[t - t0] - mx);
    sc[t - t0] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[1][wave] = sum;
  __syncthreads();
  // Weighted sum of the value rows: 16 groups of 16 threads, each thread 4
  // consecutive columns, group g takes positions t0+g, t0+g+16, ...; four
  // rows in flight per thread.
  const int grp = tid >> 4, c4 = (tid & 15) * 4;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  auto vrow = [&](int t, float (&v)[4]) {
    if (t == pos) {
      v[0] = vn[c4]; v[1] = vn[c4 + 1]; v[2] = vn[c4 + 2]; v[3] = vn[c4 + 3];
    } else {
      const E *p = cache + (size_t)t * 2 * C + C + c4;
      if constexpr (sizeof(E) == 2) {
        const uint2 u = *(const uint2 *)p;
        v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
        v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
      } else {
        const float4 u = *(const float4 *)p;
        v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
      }
    }
  };
  int t = t0 + grp;
  for (; t + 48 < t1; t += 64) {
    float v0[4], v1[4], v2[4], v3[4];
    vrow(t, v0); vrow(t + 16, v1); vrow(t + 32, v2); vrow(t + 48, v3);
    const float p0 = sc[t - t0], p1 = sc[t + 16 - t0], p2 = sc[t + 32 - t0], p3 = sc[t + 48 - t0];
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) o[q2] += (p0 * v0[q2] + p1 * v1[q2]) + (p2 * v2[q2] + p3 * v3[q2]);
  }
  for (; t < t1; t += 16) {
    float v[4];
    vrow(t, v);
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) o[q2] += sc[t - t0] * v[q2];
  }
  __shared__ float4 part[16][16];
  part[grp][tid & 15] = make_float4(o[0], o[1], o[2], o[3]);
  __syncthreads();
  if (tid < 64) {
    const int c = tid >> 2, q2 = tid & 3;
    float a = 0.f;
#pragma unroll
    for (int g = 0; g < 16; ++g) a += (&part[g][c].x)[q2];
    po[2 + c * 4 + q2] = a;
    if (tid == 0) {
      po[0] = mx;
      po[1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    }
  }
}

// att[b, h*64 + d] = sum_s w_s o_s[d] / sum_s w_s l_s with w_s = exp(m_s - m),
// m = max_s m_s (empty ranges have m_s = -inf and weigh nothing).
template <typename E>
__global__ void __launch_bounds__(64) attn_decode_combine_kernel(int NH, int S,
                                                                 const float *__restrict__ part,
                                                                 E *__restrict__ att) {
  const int bh = blockIdx.x, d = threadIdx.x;
  const float *p = part + (size_t)bh * S * DEC_PART;
  float m = -INFINITY;
  for (int s = 0; s < S; ++s) m = fmaxf(m, p[s * DEC_PART]);
  float l = 0.f, o = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ms = p[s * DEC_PART];
    const float w = ms == -INFINITY ? 0.f : __expf(ms - m);
    l += w * p[s * DEC_PART + 1];
    o += w * p[s * DEC_PART + 2 + d];
  }
  const int b = bh / NH, h = bh % NH;
  st_elem(att, (size_t)b * NH * 64 + h * 64 + d, o / l);
}

// Decode step input: the position and the tokens go to device memory, where
// the (possibly graph-replayed) step reads them.
__global__ void decode_prep_kernel(int B, int pos, const int32_t *__restrict__ tok,
                                   int32_t *__restrict__ tok_dev, int32_t *__restrict__ pos_dev) {
  const int i = threadIdx.x;
  if (i < B) tok_dev[i] = tok[i];
  if (i == 0) *pos_dev = pos;
}

// x[b] = wte[tok[b]] + wpe[pos] for the B tokens of one decode step (the
// embedding of the tinytorch page's model; out-of-range ids set the context's
// range flag and give NaN rows, as in the training embedding).
__global__ void __launch_bounds__(256) embed_decode_kernel(int B, int C, int V,
                                                           const int32_t *__restrict__ tok,
                                                           const int32_t *__restrict__ pos_p,
                                                           const float *__restrict__ wte,
                                                           const float *__restrict__ wpe,
                                                           float *__restrict__ x, int32_t *flags) {
  const int b = blockIdx.x, pos = *pos_p;
  const int id = tok[b];
  const bool ok = id >= 0 && id < V;
  if (!ok && threadIdx.x == 0) atomicOr(flags, 1);
  const float4 *w = (const float4 *)(wte + (size_t)(ok ? id : 0) * C);
  const float4 *p = (const float4 *)(wpe + (size_t)pos * C);
  float4 *o = (float4 *)(x + (size_t)b * C);
  for (int c = threadIdx.x; c < C / 4; c += 256) {
    const float4 a = w[c], e = p[c];
    o[c] = ok ? make_float4(a.x + e.x, a.y + e.y, a.z + e.z, a.w + e.w)
              : make_float4(NAN, NAN, NAN, NAN);
  }
}

__global__ void copy_i32_kernel(int n, const int32_t *__restrict__ src, int32_t *__restrict__ dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

extern "C" int tt_argmax(tt_ctx *ctx, tt_mode mode, int N, int V, int ld, const void *logits,
                         int32_t *out) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode == TT_F32 || mode == TT_BF16, "argmax: bad mode");
  TT_REQUIRE(ctx, N >= 0 && V > 0 && ld >= V, "argmax: bad shape");
  TT_REQUIRE(ctx, N == 0 || (logits && out), "argmax: NULL pointer");
  if (N == 0) return TT_OK;
  const bool bf = mode == TT_BF16;
  const bool vec = tt_aligned16(logits) && ld % (bf ? 8 : 4) == 0;
  tt_prof_scope prof(ctx, "argmax_kernel", 0.0, (double)N * V * (bf ? 2.0 : 4.0) + 4.0 * N);
  if (bf && vec)
    hipLaunchKernelGGL((argmax_kernel<true, true>), dim3(N), dim3(256), 0, ctx->stream, V, ld, logits, out);
  else if (bf)
    hipLaunchKernelGGL((argmax_kernel<true, false>), dim3(N), dim3(256), 0, ctx->stream, V, ld, logits, out);
  else if (vec)
    hipLaunchKernelGGL((argmax_kernel<false, true>), dim3(N), dim3(256), 0, ctx->stream, V, ld, logits, out);
  else
    hipLaunchKernelGGL((argmax_kernel<false, false>), dim3(N), dim3(256), 0, ctx->stream, V, ld, logits, out);
  return tt_check_launch(ctx, "argmax");
}

int tt_kv_store(tt_ctx *ctx, tt_mode mode, int B, int T, int C, int T_max, const void *qkv,
                void *kv) {
  TT_REQUIRE(ctx, B > 0 && T > 0 && T <= T_max && C % 8 == 0, "kv_store: bad shape");
  TT_REQUIRE(ctx, tt_aligned16(qkv) && tt_aligned16(kv), "kv_store: alignment");
  const size_t es = mode == TT_BF16 ? 2 : 4;
  tt_prof_scope prof(ctx, "kv_store_kernel", 0.0, 4.0 * B * T * (double)C * es);
  if (mode == TT_BF16)
    hipLaunchKernelGGL(kv_store_kernel<bf16_t>, dim3(B * T), dim3(256), 0, ctx->stream, T, C, T_max,
                       (const bf16_t *)qkv, (bf16_t *)kv);
  else
    hipLaunchKernelGGL(kv_store_kernel<float>, dim3(B * T), dim3(256), 0, ctx->stream, T, C, T_max,
                       (const float *)qkv, (float *)kv);
  return tt_check_launch(ctx, "kv_store");
}

int tt_decode_splits(int B, int NH) {
  // enough workgroups to fill the chip, at most TT_DECODE_MAX_SPLITS per (sequence, head)
  return std::max(1, std::min(TT_DECODE_MAX_SPLITS, (512 + B * NH - 1) / (B * NH)));
}

int tt_attn_decode(tt_ctx *ctx, tt_mode mode, int B, int NH, const int32_t *pos_dev, int pos_hint,
                   int T_max, const void *qkv, void *kv, void *att, float *part, int S) {
  TT_REQUIRE(ctx, B > 0 && NH > 0 && T_max <= 16384 && S >= 1 && S <= TT_DECODE_MAX_SPLITS,
             "attn_decode: bad shape");
  TT_REQUIRE(ctx, tt_aligned16(kv) && pos_dev, "attn_decode: alignment / NULL position");
  const size_t es = mode == TT_BF16 ? 2 : 4;
  const int C = NH * 64;
  const size_t lds = (size_t)((T_max + S - 1) / S) * 4;   // the longest key range
  {
    tt_prof_scope prof(ctx, "attn_decode_kernel", 4.0 * B * NH * 64.0 * (pos_hint + 1),
                       (double)B * (pos_hint + 1) * 2 * C * es + 4.0 * B * C * es);
    if (mode == TT_BF16)
      hipLaunchKernelGGL(attn_decode_kernel<bf16_t>, dim3(B * NH * S), dim3(256), lds, ctx->stream,
                         NH, pos_dev, T_max, S, (const bf16_t *)qkv, (bf16_t *)kv, part);
    else
      hipLaunchKernelGGL(attn_decode_kernel<float>, dim3(B * NH * S), dim3(256), lds, ctx->stream,
                         NH, pos_dev, T_max, S, (const float *)qkv, (float *)kv, part);
    TT_TRY(tt_check_launch(ctx, "attn_decode"));
  }
  tt_prof_scope prof(ctx, "attn_decode_combine_kernel", 0.0, 4.0 * B * NH * S * DEC_PART + B * C * es);
  if (mode == TT_BF16)
    hipLaunchKernelGGL(attn_decode_combine_kernel<bf16_t>, dim3(B * NH), dim3(64), 0, ctx->stream,
                       NH, S, part, (bf16_t *)att);
  else
    hipLaunchKernelGGL(attn_decode_combine_kernel<float>, dim3(B * NH), dim3(64), 0, ctx->stream,
                       NH, S, part, (float *)att);
  return tt_check_launch(ctx, "attn_decode_combine");
}

int tt_decode_prep(tt_ctx *ctx, int B, int pos, const int32_t *tok, int32_t *tok_dev,
                   int32_t *pos_dev) {
  TT_REQUIRE(ctx, B > 0 && B <= 1024 && tok && tok_dev && pos_dev, "decode_prep: bad arguments");
  hipLaunchKernelGGL(decode_prep_kernel, dim3(1), dim3(1024), 0, ctx->stream, B, pos, tok, tok_dev,
                     pos_dev);
  return tt_check_launch(ctx, "decode_prep");
}

int tt_embed_decode(tt_ctx *ctx, int B, int C, int V, const int32_t *tok_dev,
                    const int32_t *pos_dev, const float *wte, const float *wpe, float *x) {
  TT_REQUIRE(ctx, B > 0 && C % 4 == 0 && tt_aligned16(wte) && tt_aligned16(wpe) && tt_aligned16(x),
             "embed_decode: bad arguments");
  tt_prof_scope prof(ctx, "embed_decode_kernel", 0.0, 12.0 * B * (double)C + 8.0 * B);
  hipLaunchKernelGGL(embed_decode_kernel, dim3(B), dim3(256), 0, ctx->stream, B, C, V, tok_dev,
                     pos_dev, wte, wpe, x, ctx->dev_flags);
  return tt_check_launch(ctx, "embed_decode");
}

int tt_copy_i32(tt_ctx *ctx, int n, const int32_t *src, int32_t *dst) {
  if (n <= 0) return TT_OK;
  hipLaunchKernelGGL(copy_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, ctx->stream, n, src, dst);
  return tt_check_launch(ctx, "copy_i32");
}
