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
// scale 1/8, keys 0..pos.  One workgroup per (sequence, head): the new key and value are
// appended to the cache, the pos+1 scores go to LDS, softmax over them, then
// the output is their weighted sum of the value rows (lane = output column,
// so each value row is read coalesced).  The new position's own key and
// value are taken from the workgroup's copy, not re-read from the cache.
template <typename E>
__global__ void __launch_bounds__(256) attn_decode_kernel(int NH, int pos, int T_max,
                                                          const E *__restrict__ qkv, E *kv,
                                                          E *__restrict__ att) {
  extern __shared__ float sc[];   // [pos + 1] scores, then probabilities
  __shared__ float q[64], kn[64], vn[64];
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x / NH, h = blockIdx.x % NH;
  const int C = NH * 64;
  const E *row = qkv + (size_t)b * 3 * C + h * 64;
  E *cache = kv + (size_t)b * T_max * 2 * C + h * 64;   // key of position t at t * 2C
  if (tid < 64) {
    q[tid] = ld_elem(row, tid);
    kn[tid] = ld_elem(row + C, tid);
    vn[tid] = ld_elem(row + 2 * C, tid);
    cache[(size_t)pos * 2 * C + tid] = row[C + tid];
    cache[(size_t)pos * 2 * C + C + tid] = row[2 * C + tid];
  }
  __syncthreads();
  float mx = -INFINITY;
  for (int t = tid; t <= pos; t += 256) {
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
    sc[t] = s;
    mx = fmaxf(mx, s);
  }
  mx = wave_max(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
  __syncthreads();
  float sum = 0.f;
  for (int t = tid; t <= pos; t += 256) {
    const float e = __expf(sc[t] - mx);
    sc[t] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[1][wave] = sum;
  __syncthreads();
  const float l = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  float acc = 0.f;
  for (int t = wave; t <= pos; t += 4) {
    const float v = t == pos ? vn[lane] : ld_elem(cache + (size_t)t * 2 * C + C, lane);
    acc += sc[t] * v;
  }
  __shared__ float part[4][64];
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const float o = ((part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane])) / l;
    st_elem(att, (size_t)b * C + h * 64 + lane, o);
  }
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

int tt_attn_decode(tt_ctx *ctx, tt_mode mode, int B, int NH, int pos, int T_max, const void *qkv,
                   void *kv, void *att) {
  TT_REQUIRE(ctx, B > 0 && NH > 0 && pos >= 0 && pos < T_max && T_max <= 16384,
             "attn_decode: bad shape");
  TT_REQUIRE(ctx, tt_aligned16(kv), "attn_decode: alignment");
  const size_t es = mode == TT_BF16 ? 2 : 4;
  const int C = NH * 64;
  const size_t lds = (size_t)(pos + 1) * 4;
  tt_prof_scope prof(ctx, "attn_decode_kernel", 4.0 * B * NH * 64.0 * (pos + 1),
                     (double)B * (pos + 1) * 2 * C * es + 4.0 * B * C * es);
  if (mode == TT_BF16)
    hipLaunchKernelGGL(attn_decode_kernel<bf16_t>, dim3(B * NH), dim3(256), lds, ctx->stream, NH, pos,
                       T_max, (const bf16_t *)qkv, (bf16_t *)kv, (bf16_t *)att);
  else
    hipLaunchKernelGGL(attn_decode_kernel<float>, dim3(B * NH), dim3(256), lds, ctx->stream, NH, pos,
                       T_max, (const float *)qkv, (float *)kv, (float *)att);
  return tt_check_launch(ctx, "attn_decode");
}
