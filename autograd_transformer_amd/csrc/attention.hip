// Causal multi-head attention, forward and backward, flash style on MFMA.
//
// What is computed — tinytorch page §4 (causal mask; softmax with the row max
// subtracted) and the Forge page "最硬的一关" (scores divided by sqrt(d_k),
// -inf above the diagonal): per (batch, head), S = Q Kᵀ / sqrt(64),
// S[i, j > i] = -inf, P = softmax_row(S), O = P V; lse[i] = log sum_j exp S[i,j].
// The T x T score matrix is never stored: key blocks stream through LDS and
// the softmax is accumulated online (running max and rescaled sum).
//
// Layout trick.  An MFMA accumulator block D (16 x 16) lives as D[4g+r][c]
// in lane (g = lane/16, c = lane%16), register r.  Such a block can be fed
// straight back as the B operand of the next MFMA when the next product
// reduces over D's ROW index: lane (g, c) supplies column c, and its k slots
// hold rows 4g + r.  The A operand then reads its k values in the same
// permuted order (two 4-element runs for bf16), so sum_k is unchanged.  Hence
// the kernels compute transposed products (Sᵀ = K Qᵀ, Oᵀ = Vᵀ Pᵀ, dVᵀ = dOᵀ P,
// ...) and keep P and dS in registers.
#include "tt_internal.h"

namespace {

constexpr int HS = 64;   // head size (fixed)
constexpr int BKV = 64;  // keys per block
constexpr float LOG2E = 1.4426950408889634f;

template <typename T> struct AT;
template <> struct AT<bf16_t> {
  static constexpr int KPL = 8, KSTEP = 32, VEC = 8, PAD = 8;
  typedef bf16x8_t frag_t;
  __device__ __forceinline__ static f32x4_t mfma(frag_t a, frag_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct AT<float> {
  static constexpr int KPL = 1, KSTEP = 4, VEC = 4, PAD = 4;
  typedef float frag_t;
  __device__ __forceinline__ static f32x4_t mfma(frag_t a, frag_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

constexpr int LDT(int pad) { return HS + pad; }

__device__ __forceinline__ bf16x8_t pack8(f32x4_t a, f32x4_t b) {
  uint4 u = make_uint4(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]),
                       pack_bf2(b[2], b[3]));
  return __builtin_bit_cast(bf16x8_t, u);
}

// A-operand fragment of a row of a transposed LDS tile (row-contiguous in the
// reduction index), in the permuted slot order matching an accumulator pair:
// slots 0..3 <- cols base + 4g .. +3, slots 4..7 <- cols base + 16 + 4g .. +3.
__device__ __forceinline__ bf16x8_t perm_frag(const bf16_t *row, int base, int g) {
  uint2 lo = *(const uint2 *)(row + base + 4 * g);
  uint2 hi = *(const uint2 *)(row + base + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Cooperative copy of a 64-row x 64-col head slice into LDS, row layout
// dst[r][c] (r = token, c = head dim).  Rows >= rows_valid are zero.
template <typename T>
__device__ __forceinline__ void load_rows(T *dst, int ld_dst, const T *src, size_t ld_src, int r0,
                                          int rows_valid, int tid) {
  constexpr int VEC = AT<T>::VEC;
  constexpr int UNITS = 64 * HS / VEC;
#pragma unroll
  for (int i = 0; i < UNITS / 256; ++i) {
    int u = tid + i * 256;
    int r = u / (HS / VEC), c = (u % (HS / VEC)) * VEC;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + r < rows_valid) v = *(const uint4 *)(src + (size_t)(r0 + r) * ld_src + c);
    *(uint4 *)(dst + r * ld_dst + c) = v;
  }
}

// Same slice stored transposed: dst[c][r].
template <typename T>
__device__ __forceinline__ void load_rows_t(T *dst, int ld_dst, const T *src, size_t ld_src,
                                            int r0, int rows_valid, int tid) {
  if constexpr (sizeof(T) == 2) {
    // unit = (row pair, 8-col chunk): 32 pairs x 8 chunks = 256 units.
    int rp = tid % 32, cc = tid / 32;
    int r = 2 * rp, c = cc * 8;
    uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
    if (r0 + r < rows_valid) a = *(const uint4 *)(src + (size_t)(r0 + r) * ld_src + c);
    if (r0 + r + 1 < rows_valid) b = *(const uint4 *)(src + (size_t)(r0 + r + 1) * ld_src + c);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *(uint32_t *)(dst + (c + 2 * q) * ld_dst + r) = (aw[q] & 0xffffu) | (bw[q] << 16);
      *(uint32_t *)(dst + (c + 2 * q + 1) * ld_dst + r) = (aw[q] >> 16) | (bw[q] & 0xffff0000u);
    }
  } else {
    // unit = (row, 4-col chunk): 64 rows x 16 chunks = 1024 units, 4 per thread.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int u = tid + i * 256;
      int r = u % 64, c = (u / 64) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r0 + r < rows_valid) v = *(const float4 *)(src + (size_t)(r0 + r) * ld_src + c);
      dst[(c + 0) * ld_dst + r] = v.x;
      dst[(c + 1) * ld_dst + r] = v.y;
      dst[(c + 2) * ld_dst + r] = v.z;
      dst[(c + 3) * ld_dst + r] = v.w;
    }
  }
}

// Fragments of 16 consecutive head-dim rows of one token per lane, loaded
// from global memory: lane (g, c) gets row (tok0 + c), dims s*KSTEP + g*KPL...
template <typename T>
__device__ __forceinline__ void load_frags(typename AT<T>::frag_t *f, const T *src, size_t ld,
                                           int tok, int T_, int g) {
  constexpr int NS = HS / AT<T>::KSTEP;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if constexpr (sizeof(T) == 2) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok < T_) v = *(const uint4 *)(src + (size_t)tok * ld + s * 32 + g * 8);
      f[s] = __builtin_bit_cast(bf16x8_t, v);
    } else {
      f[s] = tok < T_ ? src[(size_t)tok * ld + s * 4 + g] : 0.f;
    }
  }
}

// ------------------------------------------------------------------ forward
// Workgroup: 4 waves x 32 queries (two 16-query column blocks per wave).
template <typename T>
__global__ void __launch_bounds__(256) attn_fwd_kernel(int T_, int NH, const T *__restrict__ qkv,
                                                       T *__restrict__ out,
                                                       float *__restrict__ lse, int nqb) {
  using A = AT<T>;
  constexpr int LD = LDT(A::PAD);
  constexpr int NS = HS / A::KSTEP;
  __shared__ __attribute__((aligned(16))) T Ks[BKV * LD];
  __shared__ __attribute__((aligned(16))) T Vt[HS * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  // heavy (late) query blocks first
  const int qb = nqb - 1 - (blockIdx.x % nqb);
  const int bh = blockIdx.x / nqb;
  const int b = bh / NH, h = bh % NH;
  const int C = NH * HS;
  const size_t ld = 3 * (size_t)C;
  const T *base = qkv + (size_t)b * T_ * ld;
  const T *Qg = base + h * HS, *Kg = base + C + h * HS, *Vg = base + 2 * C + h * HS;

  const int q0 = qb * 128 + wave * 32;
  typename A::frag_t qf[2][NS];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) load_frags<T>(qf[qs], Qg, ld, q0 + qs * 16 + c, T_, g);

  f32x4_t o[4][2];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) o[d][qs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  const float sl2 = 0.125f * LOG2E;

  const int kend = min(T_, qb * 128 + 128);
  for (int kb = 0; kb * BKV < kend; ++kb) {
    const int k0 = kb * BKV;
    __syncthreads();
    load_rows<T>(Ks, LD, Kg, ld, k0, T_, tid);
    load_rows_t<T>(Vt, LD, Vg, ld, k0, T_, tid);
    __syncthreads();
    if (k0 > q0 + 31 || q0 >= T_) continue;  // whole block masked for this wave

    f32x4_t s[4][2];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          typename A::frag_t ka =
              *(const typename A::frag_t *)(Ks + (j * 16 + c) * LD + st * A::KSTEP + g * A::KPL);
          acc = A::mfma(ka, qf[qs][st], acc);
        }
        s[j][qs] = acc;
      }
    const bool diag = k0 + BKV > q0;  // some key may exceed a query of this wave
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int q = q0 + qs * 16 + c;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + j * 16 + g * 4 + r;
          float v = s[j][qs][r] * sl2;
          if ((diag && key > q) || key >= T_) v = -INFINITY;
          s[j][qs][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qs], mx);
      const float alpha = (mrow[qs] == -INFINITY) ? 0.f : exp2f(mrow[qs] - mnew);
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float p = (s[j][qs][r] == -INFINITY) ? 0.f : exp2f(s[j][qs][r] - mnew);
          s[j][qs][r] = p;
          ps += p;
        }
      lrow[qs] = lrow[qs] * alpha + ps;
      mrow[qs] = mnew;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[d][qs][r] *= alpha;
    }
    // Oᵀ += Vᵀ Pᵀ
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const T *vrow = Vt + (d * 16 + c) * LD;
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            bf16x8_t va = perm_frag(vrow, t2 * 32, g);
            o[d][qs] = A::mfma(va, pack8(s[2 * t2][qs], s[2 * t2 + 1][qs]), o[d][qs]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              o[d][qs] = A::mfma(vrow[j * 16 + g * 4 + r], s[j][qs][r], o[d][qs]);
        }
      }
    }
  }

  // normalise and store
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    float l = lrow[qs];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int q = q0 + qs * 16 + c;
    if (q >= T_) continue;
    const float inv = 1.0f / l;
    T *orow = out + ((size_t)b * T_ + q) * C + h * HS;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int dd = d * 16 + g * 4;
      float v0 = o[d][qs][0] * inv, v1 = o[d][qs][1] * inv, v2 = o[d][qs][2] * inv,
            v3 = o[d][qs][3] * inv;
      if constexpr (sizeof(T) == 2)
        *(uint2 *)(orow + dd) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
      else
        *(float4 *)(orow + dd) = make_float4(v0, v1, v2, v3);
    }
    if (g == 0) lse[((size_t)b * NH + h) * T_ + q] = (mrow[qs] + log2f(l)) / LOG2E;
  }
}

// ------------------------------------------------------- backward helpers
// Dv[b,h,q] = sum_d dO[q, h*64+d] * O[q, h*64+d]  (= sum_j P dP, the softmax
// backward's row term).
template <typename T>
__global__ void __launch_bounds__(256) attn_bwd_dot_kernel(int BT, int T_, int NH,
                                                           const T *__restrict__ o,
                                                           const T *__restrict__ dO,
                                                           float *__restrict__ Dv) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= BT * NH) return;
  const int row = idx / NH, h = idx % NH;
  const int b = row / T_, q = row % T_;
  const size_t off = (size_t)row * NH * HS + h * HS;
  float s = 0.f;
#pragma unroll 8
  for (int d = 0; d < HS; ++d) s += Elem<T>::load(dO, off + d) * Elem<T>::load(o, off + d);
  Dv[((size_t)b * NH + h) * T_ + q] = s;
}

// dK, dV: workgroup owns 64 keys (4 waves x 16), walks query blocks from the
// diagonal to the end.  Per 16 x 16 (query, key) block, with rows = queries:
//   S = Q Kᵀ ; P = exp(S/8 - lse) ; dP = dO Vᵀ ; dS = P (dP - Dv)
//   dVᵀ += dOᵀ P ; dKᵀ += Qᵀ dS      (reductions over the query = row index)
template <typename T>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_kernel(int T_, int NH,
                                                            const T *__restrict__ qkv,
                                                            const T *__restrict__ dO,
                                                            const float *__restrict__ lse,
                                                            const float *__restrict__ Dv,
                                                            T *__restrict__ dqkv, int nkb) {
  using A = AT<T>;
  constexpr int LD = LDT(A::PAD);
  constexpr int NS = HS / A::KSTEP;
  __shared__ __attribute__((aligned(16))) T Qs[64 * LD];
  __shared__ __attribute__((aligned(16))) T dOs[64 * LD];
  __shared__ __attribute__((aligned(16))) T Qt[HS * LD];
  __shared__ __attribute__((aligned(16))) T dOt[HS * LD];
  __shared__ float lse_s[64], D_s[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int kb = blockIdx.x % nkb;
  const int bh = blockIdx.x / nkb;
  const int b = bh / NH, h = bh % NH;
  const int C = NH * HS;
  const size_t ld = 3 * (size_t)C;
  const T *base = qkv + (size_t)b * T_ * ld;
  const T *Qg = base + h * HS, *Kg = base + C + h * HS, *Vg = base + 2 * C + h * HS;
  const T *dOg = dO + (size_t)b * T_ * C + h * HS;
  const float *lseg = lse + ((size_t)b * NH + h) * T_;
  const float *Dg = Dv + ((size_t)b * NH + h) * T_;
  const float sl2 = 0.125f * LOG2E;

  const int key = kb * 64 + wave * 16 + c;  // this lane's key column
  typename A::frag_t kf[NS], vf[NS];
  load_frags<T>(kf, Kg, ld, key, T_, g);
  load_frags<T>(vf, Vg, ld, key, T_, g);

  f32x4_t dk[4], dv[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    dk[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    dv[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int nqb = (T_ + 63) / 64;
  for (int qb = kb; qb < nqb; ++qb) {
    const int q0 = qb * 64;
    __syncthreads();
    load_rows<T>(Qs, LD, Qg, ld, q0, T_, tid);
    load_rows<T>(dOs, LD, dOg, C, q0, T_, tid);
    load_rows_t<T>(Qt, LD, Qg, ld, q0, T_, tid);
    load_rows_t<T>(dOt, LD, dOg, C, q0, T_, tid);
    if (tid < 64) {
      lse_s[tid] = q0 + tid < T_ ? lseg[q0 + tid] * LOG2E : INFINITY;
      D_s[tid] = q0 + tid < T_ ? Dg[q0 + tid] : 0.f;
    }
    __syncthreads();
    if (kb * 64 + wave * 16 > q0 + 63) continue;  // all 16 keys after every query

    f32x4_t p[4], ds[4];
#pragma unroll
    for (int qs = 0; qs < 4; ++qs) {
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f}, dpacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int off = (qs * 16 + c) * LD + st * A::KSTEP + g * A::KPL;
        sacc = A::mfma(*(const typename A::frag_t *)(Qs + off), kf[st], sacc);
        dpacc = A::mfma(*(const typename A::frag_t *)(dOs + off), vf[st], dpacc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ql = qs * 16 + g * 4 + r;
        const int q = q0 + ql;
        float pv = (key > q || q >= T_ || key >= T_) ? 0.f : exp2f(sacc[r] * sl2 - lse_s[ql]);
        p[qs][r] = pv;
        ds[qs][r] = pv * (dpacc[r] - D_s[ql]);
      }
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const T *qrow = Qt + (d * 16 + c) * LD;
      const T *orow = dOt + (d * 16 + c) * LD;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          dv[d] = A::mfma(perm_frag(orow, t2 * 32, g), pack8(p[2 * t2], p[2 * t2 + 1]), dv[d]);
          dk[d] = A::mfma(perm_frag(qrow, t2 * 32, g), pack8(ds[2 * t2], ds[2 * t2 + 1]), dk[d]);
        }
      } else {
#pragma unroll
        for (int qs = 0; qs < 4; ++qs)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dv[d] = A::mfma(orow[qs * 16 + g * 4 + r], p[qs][r], dv[d]);
            dk[d] = A::mfma(qrow[qs * 16 + g * 4 + r], ds[qs][r], dk[d]);
          }
      }
    }
  }
  if (key >= T_) return;
  T *drow = dqkv + ((size_t)b * T_ + key) * ld + h * HS;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int dd = d * 16 + g * 4;
    float k0 = dk[d][0] * 0.125f, k1 = dk[d][1] * 0.125f, k2 = dk[d][2] * 0.125f,
          k3 = dk[d][3] * 0.125f;
    if constexpr (sizeof(T) == 2) {
      *(uint2 *)(drow + C + dd) = make_uint2(pack_bf2(k0, k1), pack_bf2(k2, k3));
      *(uint2 *)(drow + 2 * C + dd) =
          make_uint2(pack_bf2(dv[d][0], dv[d][1]), pack_bf2(dv[d][2], dv[d][3]));
    } else {
      *(float4 *)(drow + C + dd) = make_float4(k0, k1, k2, k3);
      *(float4 *)(drow + 2 * C + dd) = make_float4(dv[d][0], dv[d][1], dv[d][2], dv[d][3]);
    }
  }
}

// dQ: workgroup owns 64 queries (4 waves x 16), walks key blocks up to the
// diagonal.  Per block, with rows = keys (transposed):
//   Sᵀ = K Qᵀ ; Pᵀ ; dPᵀ = V dOᵀ ; dSᵀ = Pᵀ (dPᵀ - Dv) ; dQᵀ += Kᵀ dSᵀ.
template <typename T>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(int T_, int NH,
                                                          const T *__restrict__ qkv,
                                                          const T *__restrict__ dO,
                                                          const float *__restrict__ lse,
                                                          const float *__restrict__ Dv,
                                                          T *__restrict__ dqkv, int nqb) {
  using A = AT<T>;
  constexpr int LD = LDT(A::PAD);
  constexpr int NS = HS / A::KSTEP;
  __shared__ __attribute__((aligned(16))) T Ks[64 * LD];
  __shared__ __attribute__((aligned(16))) T Vs[64 * LD];
  __shared__ __attribute__((aligned(16))) T Kt[HS * LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int qb = nqb - 1 - (blockIdx.x % nqb);
  const int bh = blockIdx.x / nqb;
  const int b = bh / NH, h = bh % NH;
  const int C = NH * HS;
  const size_t ld = 3 * (size_t)C;
  const T *base = qkv + (size_t)b * T_ * ld;
  const T *Qg = base + h * HS, *Kg = base + C + h * HS, *Vg = base + 2 * C + h * HS;
  const T *dOg = dO + (size_t)b * T_ * C + h * HS;
  const float sl2 = 0.125f * LOG2E;

  const int q = qb * 64 + wave * 16 + c;  // this lane's query column
  typename A::frag_t qf[NS], of[NS];
  load_frags<T>(qf, Qg, ld, q, T_, g);
  load_frags<T>(of, dOg, C, q, T_, g);
  const float lq = q < T_ ? lse[((size_t)b * NH + h) * T_ + q] * LOG2E : 0.f;
  const float Dq = q < T_ ? Dv[((size_t)b * NH + h) * T_ + q] : 0.f;

  f32x4_t dq[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) dq[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kend = min(T_, qb * 64 + 64);
  const int qw0 = qb * 64 + wave * 16;
  for (int kb = 0; kb * 64 < kend; ++kb) {
    const int k0 = kb * 64;
    __syncthreads();
    load_rows<T>(Ks, LD, Kg, ld, k0, T_, tid);
    load_rows<T>(Vs, LD, Vg, ld, k0, T_, tid);
    load_rows_t<T>(Kt, LD, Kg, ld, k0, T_, tid);
    __syncthreads();
    if (k0 > qw0 + 15) continue;
    f32x4_t ds[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f}, dpacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int off = (j * 16 + c) * LD + st * A::KSTEP + g * A::KPL;
        sacc = A::mfma(*(const typename A::frag_t *)(Ks + off), qf[st], sacc);
        dpacc = A::mfma(*(const typename A::frag_t *)(Vs + off), of[st], dpacc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + j * 16 + g * 4 + r;
        float pv = (key > q || key >= T_ || q >= T_) ? 0.f : exp2f(sacc[r] * sl2 - lq);
        ds[j][r] = pv * (dpacc[r] - Dq);
      }
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const T *krow = Kt + (d * 16 + c) * LD;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          dq[d] = A::mfma(perm_frag(krow, t2 * 32, g), pack8(ds[2 * t2], ds[2 * t2 + 1]), dq[d]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) dq[d] = A::mfma(krow[j * 16 + g * 4 + r], ds[j][r], dq[d]);
      }
    }
  }
  if (q >= T_) return;
  T *drow = dqkv + ((size_t)b * T_ + q) * ld + h * HS;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int dd = d * 16 + g * 4;
    float v0 = dq[d][0] * 0.125f, v1 = dq[d][1] * 0.125f, v2 = dq[d][2] * 0.125f,
          v3 = dq[d][3] * 0.125f;
    if constexpr (sizeof(T) == 2)
      *(uint2 *)(drow + dd) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
    else
      *(float4 *)(drow + dd) = make_float4(v0, v1, v2, v3);
  }
}

template <typename T>
int attn_fwd_t(tt_ctx *ctx, int B, int T_, int NH, const void *qkv, void *out, float *lse) {
  const int nqb = (T_ + 127) / 128;
  hipLaunchKernelGGL(attn_fwd_kernel<T>, dim3(B * NH * nqb), dim3(256), 0, ctx->stream, T_, NH,
                     (const T *)qkv, (T *)out, lse, nqb);
  return tt_check_launch(ctx, "attn_fwd");
}

template <typename T>
int attn_bwd_t(tt_ctx *ctx, int B, int T_, int NH, const void *qkv, const void *out,
               const float *lse, const void *dout, void *dqkv, float *Dv) {
  const int BT = B * T_;
  hipLaunchKernelGGL(attn_bwd_dot_kernel<T>, dim3((BT * NH + 255) / 256), dim3(256), 0,
                     ctx->stream, BT, T_, NH, (const T *)out, (const T *)dout, Dv);
  TT_TRY(tt_check_launch(ctx, "attn_bwd_dot"));
  const int nb = (T_ + 63) / 64;
  hipLaunchKernelGGL(attn_bwd_dkdv_kernel<T>, dim3(B * NH * nb), dim3(256), 0, ctx->stream, T_, NH,
                     (const T *)qkv, (const T *)dout, lse, Dv, (T *)dqkv, nb);
  TT_TRY(tt_check_launch(ctx, "attn_bwd_dkdv"));
  hipLaunchKernelGGL(attn_bwd_dq_kernel<T>, dim3(B * NH * nb), dim3(256), 0, ctx->stream, T_, NH,
                     (const T *)qkv, (const T *)dout, lse, Dv, (T *)dqkv, nb);
  return tt_check_launch(ctx, "attn_bwd_dq");
}

}  // namespace

int tt_attn_fwd_impl(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, const void *qkv, void *out,
                     float *lse) {
  if (mode == TT_BF16 && tt_attn_bf16_ok(B, T, NH)) return tt_attn_fwd_bf16(ctx, B, T, NH, qkv, out, lse);
  if (mode == TT_BF16) return attn_fwd_t<bf16_t>(ctx, B, T, NH, qkv, out, lse);
  if (mode == TT_FP16) {
    if (!tt_attn_bf16_ok(B, T, NH))
      return tt_set_error(ctx, TT_EUNSUPPORTED, "attention(fp16): qkv of 2 GB or more");
    return tt_attn_fwd_bf16(ctx, B, T, NH, qkv, out, lse, true);
  }
  return attn_fwd_t<float>(ctx, B, T, NH, qkv, out, lse);
}

int tt_attn_bwd_impl(tt_ctx *ctx, tt_mode mode, int B, int T, int NH, const void *qkv,
                     const void *out, const float *lse, const void *dout, void *dqkv, float *Dv,
                     float *dbias) {
  if (tt_lowp(mode) && tt_attn_bf16_ok(B, T, NH))
    return tt_attn_bwd_bf16(ctx, B, T, NH, qkv, out, lse, dout, dqkv, Dv, mode == TT_FP16, dbias);
  if (mode == TT_FP16)
    return tt_set_error(ctx, TT_EUNSUPPORTED, "attention(fp16): qkv of 2 GB or more");
  if (mode == TT_BF16)
    TT_TRY(attn_bwd_t<bf16_t>(ctx, B, T, NH, qkv, out, lse, dout, dqkv, Dv));
  else
    TT_TRY(attn_bwd_t<float>(ctx, B, T, NH, qkv, out, lse, dout, dqkv, Dv));
  const int C3 = 3 * NH * 64;
  return dbias ? tt_colsum(ctx, mode, B * T, C3, C3, dqkv, dbias) : TT_OK;
}
