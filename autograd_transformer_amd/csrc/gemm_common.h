// Shared pieces of the GEMM kernels: launch parameters and the epilogue.
#pragma once

#include "tt_internal.h"

namespace tt_gemm_detail {

struct GemmParams {
  const void *A; int lda;
  const void *B; int ldb;
  int M, N, K;
  int k_chunk;   // K range per split (multiple of BK)
  int epi;
  void *out; int ldo; int out_bf16;
  const float *bias;
  const float *resid; int ldr;
  void *aux; int ldx;
  int n_valid;
  int tiles_m, tiles_n;
  int vec_out;   // output/aux/resid rows allow 4-wide vector access
  uint32_t a_bytes, b_bytes;  // operand extents for buffer range checks
  size_t out_zstride;         // split-K partials: output offset per blockIdx.z (elements)
  float *colsum;              // nullable: += column sums of the stored output (v3 kernel)
  int raster_n;               // tile order: 1 = n fastest (share A panels), 0 = m fastest
  const GemmGroupEntry *group;   // grouped launch: problem table (device), else null
  const uint16_t *group_map;     // grouped launch: workgroup -> table entry
};

// Vector stores of a product's outputs: streaming (non-temporal) stores,
// which the L2 keeps at the front of its eviction order, so the tiles being
// written do not push the operand panels that other workgroups still read
// out of L2 (measured: 1.6 % off the GPT-2 124M step).
__device__ __forceinline__ void out_store(void *dst, uint2 v) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  __builtin_nontemporal_store(u32x2_t{v.x, v.y}, (u32x2_t *)dst);
}
__device__ __forceinline__ void out_store(void *dst, float4 v) {
  typedef float f32x4v_t __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(f32x4v_t{v.x, v.y, v.z, v.w}, (f32x4v_t *)dst);
}

// out_bf16: the output is 16-bit (bf16, or binary16 when F16).
template <bool F16 = false>
__device__ __forceinline__ void store_out(void *out, int ldo, int out_bf16, int m, int n, float v) {
  if (out_bf16)
    ((bf16_t *)out)[(size_t)m * ldo + n] = lp_from<F16>(v);
  else
    ((float *)out)[(size_t)m * ldo + n] = v;
}

// Epilogue for 4 consecutive columns n..n+3 of row m (only the first `cnt`
// of them exist when the tile sticks out of the matrix).  Vector accesses
// need 16-byte (f32) / 8-byte (bf16) aligned rows, which the host checks
// (p.vec_out); otherwise elements are handled one by one.  Returns the values
// as stored for EPI_STORE / EPI_GELU_BWD (bf16-rounded when the output is
// bf16, 0 past cnt), for column sums.
template <bool F16>
__device__ __forceinline__ float4 round_stored(const GemmParams &p, const float *a, int lim) {
  float r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    r[q] = q < lim ? (p.out_bf16 ? lp_to<F16>(lp_from<F16>(a[q])) : a[q]) : 0.f;
  return make_float4(r[0], r[1], r[2], r[3]);
}

template <bool F16 = false>
__device__ __forceinline__ float4 epilogue4(const GemmParams &p, int m, int n, float4 v, int cnt) {
  const bool full = cnt >= 4 && p.vec_out;
  float a[4] = {v.x, v.y, v.z, v.w};
  const int lim = cnt < 4 ? cnt : 4;
  switch (p.epi) {
    case EPI_STORE:
    case EPI_GELU: {
      if (p.epi == EPI_GELU) {
        if (p.aux) {
          if (full && p.out_bf16)
            out_store((bf16_t *)p.aux + (size_t)m * p.ldx + n,
                      make_uint2(lp_pack2<F16>(a[0], a[1]), lp_pack2<F16>(a[2], a[3])));
          else
            for (int q = 0; q < lim; ++q) store_out<F16>(p.aux, p.ldx, p.out_bf16, m, n + q, a[q]);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) a[q] = gelu_f(a[q]);
      }
      if (full) {
        if (p.out_bf16)
          out_store((bf16_t *)p.out + (size_t)m * p.ldo + n,
                    make_uint2(lp_pack2<F16>(a[0], a[1]), lp_pack2<F16>(a[2], a[3])));
        else
          out_store((float *)p.out + (size_t)m * p.ldo + n, make_float4(a[0], a[1], a[2], a[3]));
      } else {
        for (int q = 0; q < lim; ++q) store_out<F16>(p.out, p.ldo, p.out_bf16, m, n + q, a[q]);
      }
      return round_stored<F16>(p, a, lim);
    }
    case EPI_RESID: {
      const float *rp = p.resid + (size_t)m * p.ldr + n;
      float *op = (float *)p.out + (size_t)m * p.ldo + n;
      if (full) {
        float4 r = *(const float4 *)rp;
        out_store(op, make_float4(r.x + a[0], r.y + a[1], r.z + a[2], r.w + a[3]));
      } else {
        for (int q = 0; q < lim; ++q) op[q] = rp[q] + a[q];
      }
      break;
    }
    case EPI_GELU_BWD: {
      float h[4];
      if (p.out_bf16) {
        const bf16_t *hp = (const bf16_t *)p.aux + (size_t)m * p.ldx + n;
        if (full) {
          uint2 u = *(const uint2 *)hp;
          h[0] = lp_lo<F16>(u.x); h[1] = lp_hi<F16>(u.x);
          h[2] = lp_lo<F16>(u.y); h[3] = lp_hi<F16>(u.y);
        } else {
          for (int q = 0; q < 4; ++q) h[q] = q < lim ? lp_to<F16>(hp[q]) : 0.f;
        }
      } else {
        const float *hp = (const float *)p.aux + (size_t)m * p.ldx + n;
        for (int q = 0; q < 4; ++q) h[q] = q < lim ? hp[q] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] *= gelu_grad_f(h[q]);
      if (full && p.out_bf16)
        out_store((bf16_t *)p.out + (size_t)m * p.ldo + n,
                  make_uint2(lp_pack2<F16>(a[0], a[1]), lp_pack2<F16>(a[2], a[3])));
      else
        for (int q = 0; q < lim; ++q) store_out<F16>(p.out, p.ldo, p.out_bf16, m, n + q, a[q]);
      return round_stored<F16>(p, a, lim);
    }
    case EPI_ACCUM: {
      float *op = (float *)p.out + (size_t)m * p.ldo + n;
      for (int q = 0; q < lim; ++q) unsafeAtomicAdd(op + q, a[q]);
      break;
    }
    case EPI_STORE_ACC: {
      float *op = (float *)p.out + (size_t)m * p.ldo + n;
      for (int q = 0; q < lim; ++q) op[q] += a[q];
      break;
    }
  }
  return make_float4(0.f, 0.f, 0.f, 0.f);
}


// Block id -> (tile_m, tile_n).  Workgroups are dispatched round-robin over
// the 8 XCDs (each with its own L2), so first give every XCD a contiguous
// range of tiles, then walk that range in groups of G tile-rows (m fastest:
// consecutive workgroups share B panels) or, with raster_n, of G tile-columns
// (n fastest: they share A panels), whichever operand is larger.
__device__ __forceinline__ void tile_coords(int bid, int nwg, int tiles_m, int tiles_n,
                                            int raster_n, int &tm, int &tn, bool xcd = true) {
  constexpr int XCDS = 8, G = 8;
  if (xcd && nwg % XCDS == 0) bid = (bid % XCDS) * (nwg / XCDS) + bid / XCDS;
  const int major = raster_n ? tiles_n : tiles_m, minor = raster_n ? tiles_m : tiles_n;
  const int per_group = G * minor;
  const int group = bid / per_group;
  const int first = group * G;
  const int g = min(G, major - first);
  const int in = bid % per_group;
  const int a = first + in % g, b = in / g;
  tm = raster_n ? b : a;
  tn = raster_n ? a : b;
}

// Host: may the epilogue use 4-wide vector accesses on out / aux / resid?
inline bool gemm_vec_out(const GemmArgs &g) {
  const int oes = g.out_bf16 ? 2 : 4;   // bytes per output element (aux has the same)
  bool ok = ((uintptr_t)g.out % (4 * oes) == 0) && (g.ldo % 4 == 0);
  if (g.aux) ok = ok && ((uintptr_t)g.aux % (4 * oes) == 0) && (g.ldx % 4 == 0);
  if (g.resid) ok = ok && ((uintptr_t)g.resid % 16 == 0) && (g.ldr % 4 == 0);
  if (g.epi == EPI_RESID || g.epi == EPI_ACCUM || g.epi == EPI_STORE_ACC)
    ok = ok && ((uintptr_t)g.out % 16 == 0);
  return ok;
}

// Algorithmic HBM bytes of one product (bf16 operands read once, the output
// written once, the epilogue's second input read once): with the FLOPs, the
// arithmetic intensity that says which roofline bounds the launch.
inline double gemm_bytes(const GemmArgs &g) {
  const double mn = (double)g.M * g.N;
  double b = 2.0 * ((double)g.M * g.K + (double)g.K * g.N) + mn * (g.out_bf16 ? 2.0 : 4.0);
  if (g.epi == EPI_GELU && g.aux) b += mn * (g.out_bf16 ? 2.0 : 4.0);
  if (g.epi == EPI_GELU_BWD) b += mn * (g.out_bf16 ? 2.0 : 4.0);
  if (g.epi == EPI_RESID || g.epi == EPI_STORE_ACC || (g.epi == EPI_ACCUM && !g.overwrite))
    b += mn * 4.0;
  return b;
}

// Bytes spanned by an operand: rows x reduction, k-major or row-major,
// rounded up to whole dwords.  The buffer range check works per dword: an
// extent ending inside a dword would read that dword -- and so the operand's
// last element -- as 0.  The rounding can add an element only to a row-major
// operand (k-major operands of the fast kernels have K and ld multiples of
// 8): column `rows` of its last k row, which reaches only an output that is
// not stored.
__host__ __device__ inline size_t gemm_extent_bytes(bool kmajor, int rows, int K, int ld) {
  const size_t elems = kmajor ? (size_t)(rows - 1) * ld + K : (size_t)(K - 1) * ld + rows;
  return ((elems + 1) & ~(size_t)1) * 2;
}

}  // namespace tt_gemm_detail
