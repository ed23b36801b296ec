// Bandwidth-bound kernels: LayerNorm forward/backward, fused softmax +
// cross-entropy, column sums (bias gradients).  One wave (64 lanes) owns a
// row; row statistics are wave-shuffle reductions; loads are 16-byte vectors.
#include <algorithm>

#include "tt_internal.h"

namespace {

// LN_MAXV: float4 per lane (template); C <= 64 * 4 * LN_MAXV, at most 4096.

// LayerNorm forward — tinytorch page §4 (subtract the mean, divide by the
// standard deviation, scale by the weight, add the bias); biased variance,
// eps inside the square root.  Two-pass statistics from registers.
template <bool OUT_BF16, int LN_MAXV, bool F16 = false>
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
  // every load of the row is issued before the first use (a lane past the
  // row end reads the row's last vector and contributes zero): one memory
  // round trip, where a load under a branch would wait for each in turn
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) v[i] = xr[min(lane + i * 64, nv - 1)];
#pragma unroll
  for (int i = 0; i < LN_MAXV; ++i) {
    if (lane + i * 64 >= nv) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
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
        uint2 pk = make_uint2(lp_pack2<F16>(o0, o1), lp_pack2<F16>(o2, o3));
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
// LayerNorm backward: lnb_rpw rows per wave with all of a wave's row loads
// issued before any arithmetic.  Column partials of dgamma = sum dy * xhat,
// dbeta = sum dy and the column sums of the produced dx (as stored:
// bf16-rounded when a bf16 copy is written) go to a per-wave LDS slice
// (plain stores: LDS float atomics are far slower), are summed over the
// workgroup's waves and written to part[blockIdx.x][3][C];
// layernorm_bwd_reduce_kernel then adds the workgroups' partials up.
constexpr uint32_t LN_OOB = 0x7ffffff0u;   // past every range below
// p and bytes must be wave-uniform; readfirstlane makes that visible to the
// compiler (a resource it believes divergent costs a waterfall loop per load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ln_rsrc(const float *p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ float4 ln_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// waves per workgroup and rows per wave by row width (NV float4 per lane):
// the LDS slices (waves x 3 x NV*64 float4) stay within 160 KB.
__host__ __device__ constexpr int lnb_waves(int nv) { return nv <= 4 ? 4 : (nv <= 8 ? 2 : 1); }
__host__ __device__ constexpr int lnb_rpw(int nv) { return nv <= 3 ? 2 : 1; }

template <int NV, bool F16 = false>
__global__ void __launch_bounds__(64 * lnb_waves(NV)) layernorm_bwd_kernel(
    int N, int C, const float *__restrict__ x, const float *__restrict__ mean,
    const float *__restrict__ rstd, const float *__restrict__ gamma, const float *__restrict__ dy,
    const float *dres, float *dx, bf16_t *__restrict__ dx_bf16, float *__restrict__ part) {
  constexpr int LNB_WAVES = lnb_waves(NV);
  __shared__ float4 red[LNB_WAVES][3][NV * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nv = C >> 2;
  const float4 *g4 = (const float4 *)gamma;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  const float inv_c = 1.0f / (float)C;
  constexpr int LNB_RPW = lnb_rpw(NV);
  float4 pg[NV], pb[NV], ps[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    pg[i] = z4; pb[i] = z4; ps[i] = z4;
  }
  // wave-uniform (readfirstlane: the compiler cannot see that threadIdx.x >> 6
  // is uniform, and a per-lane buffer resource would need a waterfall loop)
  const int rbase = __builtin_amdgcn_readfirstlane((blockIdx.x * LNB_WAVES + wave) * LNB_RPW);
  // Branch-free loads: buffer resources spanning this wave's valid rows;
  // columns past C take an out-of-range offset and read zero.
  const int nrows = max(0, min(LNB_RPW, N - rbase));
  const size_t base = (size_t)rbase * C;
  const uint32_t bytes = (uint32_t)nrows * C * 4;
  const __amdgpu_buffer_rsrc_t rx = ln_rsrc(x + base, bytes), rd = ln_rsrc(dy + base, bytes),
                               rr = ln_rsrc(dres ? dres + base : x, dres ? bytes : 0u);
  float4 xv[LNB_RPW][NV], dv[LNB_RPW][NV], rv[LNB_RPW][NV];
  float mu[LNB_RPW], rs[LNB_RPW];
#pragma unroll
  for (int r = 0; r < LNB_RPW; ++r) {
    const int row = min(rbase + r, N - 1);
    mu[r] = mean[row];
    rs[r] = rstd[row];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + i * 64;
      const uint32_t off = c < nv ? (uint32_t)(r * C + 4 * c) * 4u : LN_OOB;
      xv[r][i] = ln_load4(rx, off);
      dv[r][i] = ln_load4(rd, off);
      rv[r][i] = ln_load4(rr, off);
    }
  }
#pragma unroll
  for (int r = 0; r < LNB_RPW; ++r) {
    const int row = rbase + r;
    if (row >= N) break;
    float4 xh[NV], gg[NV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float4 d = dv[r][i];
      const float4 xq = xv[r][i];
      const float4 ga = lane + i * 64 < nv ? g4[lane + i * 64] : z4;   // cached
      xh[i] = make_float4((xq.x - mu[r]) * rs[r], (xq.y - mu[r]) * rs[r], (xq.z - mu[r]) * rs[r],
                          (xq.w - mu[r]) * rs[r]);
      gg[i] = make_float4(d.x * ga.x, d.y * ga.y, d.z * ga.z, d.w * ga.w);
      s1 += (gg[i].x + gg[i].y) + (gg[i].z + gg[i].w);
      s2 += (gg[i].x * xh[i].x + gg[i].y * xh[i].y) + (gg[i].z * xh[i].z + gg[i].w * xh[i].w);
      pg[i].x += d.x * xh[i].x; pg[i].y += d.y * xh[i].y;
      pg[i].z += d.z * xh[i].z; pg[i].w += d.w * xh[i].w;
      pb[i].x += d.x; pb[i].y += d.y; pb[i].z += d.z; pb[i].w += d.w;
    }
    const float m1 = wave_sum(s1) * inv_c;
    const float m2 = wave_sum(s2) * inv_c;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + i * 64;
      if (c < nv) {
        float4 o;
        o.x = rs[r] * (gg[i].x - m1 - xh[i].x * m2) + rv[r][i].x;
        o.y = rs[r] * (gg[i].y - m1 - xh[i].y * m2) + rv[r][i].y;
        o.z = rs[r] * (gg[i].z - m1 - xh[i].z * m2) + rv[r][i].z;
        o.w = rs[r] * (gg[i].w - m1 - xh[i].w * m2) + rv[r][i].w;
        ((float4 *)dx)[(size_t)row * nv + c] = o;
        if (dx_bf16) {
          const uint32_t lo = lp_pack2<F16>(o.x, o.y), hi = lp_pack2<F16>(o.z, o.w);
          ((uint2 *)dx_bf16)[(size_t)row * nv + c] = make_uint2(lo, hi);
          o = make_float4(lp_lo<F16>(lo), lp_hi<F16>(lo), lp_lo<F16>(hi), lp_hi<F16>(hi));
        }
        ps[i].x += o.x; ps[i].y += o.y; ps[i].z += o.z; ps[i].w += o.w;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + i * 64;
    red[wave][0][c] = pg[i];
    red[wave][1][c] = pb[i];
    red[wave][2][c] = ps[i];
  }
  __syncthreads();
  float4 *out = (float4 *)(part + (size_t)blockIdx.x * 3 * C);
  for (int f = threadIdx.x; f < 3 * nv; f += 64 * LNB_WAVES) {
    const int k = f / nv, c = f % nv;
    float4 a = red[0][k][c];
#pragma unroll
    for (int w = 1; w < LNB_WAVES; ++w) {
      const float4 b = red[w][k][c];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    out[f] = a;
  }
}

// LayerNorm backward for rows of at most 1024 columns (NV <= 4): the same
// arithmetic and partial-sum layout as above, but each wave walks a strided
// list of rows with two rows' loads in flight while it computes and stores
// the one before them, so a workgroup's reads and writes overlap (the
// one-round kernel above reads every row of the grid, then writes them all).
// Workgroup g owns rows [g R, (g + 1) R), R = 4 RPW; wave w takes rows
// g R + w, g R + w + 4, ... (RPW of them).  The walk is unrolled and has no
// branches (rows past the workgroup's end read zero, contribute zero and their
// stores fall outside the buffer range), so the compiler sees straight-line
// code and waits, before each row, only for that row's own loads.
constexpr int LNP_WAVES = 4;
constexpr int LNP_MAX_WG = 512;   // two workgroups per CU

// rows per wave: the smallest of 2, 4, 8 that keeps the grid within
// LNP_MAX_WG workgroups (8 beyond that)
__host__ __device__ constexpr int lnp_rpw(int N) {
  return N <= LNP_MAX_WG * LNP_WAVES * 2 ? 2 : (N <= LNP_MAX_WG * LNP_WAVES * 4 ? 4 : 8);
}

typedef uint32_t v4u32_t __attribute__((ext_vector_type(4)));
typedef uint32_t v2u32_t __attribute__((ext_vector_type(2)));

template <int NV>
struct LnRow {
  float4 x[NV], d[NV], r[NV];
  float mu, rs;
};

template <int NV, int RPW, bool F16 = false>
__global__ void __launch_bounds__(64 * LNP_WAVES) layernorm_bwd_pipe_kernel(
    int N, int C, const float *__restrict__ x, const float *__restrict__ mean,
    const float *__restrict__ rstd, const float *__restrict__ gamma, const float *__restrict__ dy,
    const float *dres, float *dx, bf16_t *__restrict__ dx_bf16, float *__restrict__ part) {
  __shared__ float4 red[LNP_WAVES][3][NV * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nv = C >> 2;
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  const float inv_c = 1.0f / (float)C;
  const int r0 = blockIdx.x * (RPW * LNP_WAVES), r1 = min(N, r0 + RPW * LNP_WAVES);
  // one resource per tensor over the workgroup's rows; columns past C and
  // rows past r1 take an out-of-range offset and read zero
  const size_t base = (size_t)r0 * C;
  const uint32_t bytes = (uint32_t)max(0, r1 - r0) * C * 4;
  const __amdgpu_buffer_rsrc_t rx = ln_rsrc(x + base, bytes), rd = ln_rsrc(dy + base, bytes),
                               rr = ln_rsrc(dres ? dres + base : x, dres ? bytes : 0u),
                               wx = ln_rsrc(dx + base, bytes);
  // the bf16 copy's resource has no range when there is no copy: its stores drop
  const __amdgpu_buffer_rsrc_t wb =
      ln_rsrc(dx_bf16 ? (const float *)(dx_bf16 + base) : dx, dx_bf16 ? bytes / 2 : 0u);
  float4 ga[NV], pg[NV], pb[NV], ps[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + i * 64;
    ga[i] = c < nv ? ((const float4 *)gamma)[c] : z4;
    pg[i] = z4; pb[i] = z4; ps[i] = z4;
  }
  auto issue = [&](LnRow<NV> &t, int row) {
    const bool ok = row < r1;
    const int lrow = row - r0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + i * 64;
      const uint32_t off = ok && c < nv ? (uint32_t)(lrow * C + 4 * c) * 4u : LN_OOB;
      t.x[i] = ln_load4(rx, off);
      t.d[i] = ln_load4(rd, off);
      t.r[i] = ln_load4(rr, off);
    }
    const int rc = min(row, N - 1);
    t.mu = mean[rc];
    t.rs = rstd[rc];
  };
  auto process = [&](const LnRow<NV> &t, int row) {
    float4 xh[NV], gg[NV];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float4 d = t.d[i], xq = t.x[i];
      xh[i] = make_float4((xq.x - t.mu) * t.rs, (xq.y - t.mu) * t.rs, (xq.z - t.mu) * t.rs,
                          (xq.w - t.mu) * t.rs);
      gg[i] = make_float4(d.x * ga[i].x, d.y * ga[i].y, d.z * ga[i].z, d.w * ga[i].w);
      s1 += (gg[i].x + gg[i].y) + (gg[i].z + gg[i].w);
      s2 += (gg[i].x * xh[i].x + gg[i].y * xh[i].y) + (gg[i].z * xh[i].z + gg[i].w * xh[i].w);
      pg[i].x += d.x * xh[i].x; pg[i].y += d.y * xh[i].y;
      pg[i].z += d.z * xh[i].z; pg[i].w += d.w * xh[i].w;
      pb[i].x += d.x; pb[i].y += d.y; pb[i].z += d.z; pb[i].w += d.w;
    }
    const float m1 = wave_sum(s1) * inv_c;
    const float m2 = wave_sum(s2) * inv_c;
    // branch-free stores: columns past C take an out-of-range offset (and
    // their partial-sum lanes are never written out)
    const int lrow = row - r0;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = lane + i * 64;
      const bool cok = c < nv;
      float4 o;
      o.x = t.rs * (gg[i].x - m1 - xh[i].x * m2) + t.r[i].x;
      o.y = t.rs * (gg[i].y - m1 - xh[i].y * m2) + t.r[i].y;
      o.z = t.rs * (gg[i].z - m1 - xh[i].z * m2) + t.r[i].z;
      o.w = t.rs * (gg[i].w - m1 - xh[i].w * m2) + t.r[i].w;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, o), wx,
                                             cok ? (uint32_t)(lrow * C + 4 * c) * 4u : LN_OOB, 0, 0);
      const uint32_t lo = lp_pack2<F16>(o.x, o.y), hi = lp_pack2<F16>(o.z, o.w);
      v2u32_t pk = {lo, hi};
      __builtin_amdgcn_raw_buffer_store_b64(pk, wb, cok ? (uint32_t)(lrow * C + 4 * c) * 2u : LN_OOB,
                                            0, 0);
      // column sums of dx as stored (the bf16 copy when there is one)
      if (dx_bf16) o = make_float4(lp_lo<F16>(lo), lp_hi<F16>(lo), lp_lo<F16>(hi), lp_hi<F16>(hi));
      ps[i].x += o.x; ps[i].y += o.y; ps[i].z += o.z; ps[i].w += o.w;
    }
  };
  LnRow<NV> t[RPW];
  const int row = r0 + wave;
  issue(t[0], row);
  if constexpr (RPW > 1) issue(t[1], row + LNP_WAVES);
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    process(t[k], row + k * LNP_WAVES);
    if (k + 2 < RPW) issue(t[k + 2], row + (k + 2) * LNP_WAVES);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + i * 64;
    red[wave][0][c] = pg[i];
    red[wave][1][c] = pb[i];
    red[wave][2][c] = ps[i];
  }
  __syncthreads();
  float4 *out = (float4 *)(part + (size_t)blockIdx.x * 3 * C);
  for (int f = threadIdx.x; f < 3 * nv; f += 64 * LNP_WAVES) {
    const int k = f / nv, c = f % nv;
    float4 a = red[0][k][c];
#pragma unroll
    for (int w = 1; w < LNP_WAVES; ++w) {
      const float4 b = red[w][k][c];
      a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
    }
    out[f] = a;
  }
}

// out_k[c] += sum_g part[g][k][c] for k = 0 (dgamma), 1 (dbeta), 2 (dx
// column sums); a NULL output is skipped.  Thread: one float4 of the [3][C]
// partial row, one of 4 row groups of a 32-row slice of the partials; LDS
// combines the groups, then one atomic per element and slice.
constexpr int LNR_SLICE = 32;

__device__ __forceinline__ void ln_reduce_body(int G, int C, const float *__restrict__ part,
                                               float *dg, float *db, float *dsum) {
  const int nf = 3 * C / 4;
  const int f = blockIdx.x * 64 + (threadIdx.x & 63);
  const int grp = threadIdx.x >> 6;
  const int g0 = blockIdx.y * LNR_SLICE, g1 = min(G, g0 + LNR_SLICE);
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (f < nf)
    for (int g = g0 + grp; g < g1; g += 4) {
      const float4 v = ((const float4 *)(part + (size_t)g * 3 * C))[f];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  __shared__ float4 red[4][64];
  red[grp][threadIdx.x & 63] = s;
  __syncthreads();
  if (grp != 0 || f >= nf) return;
  const float4 a = red[0][threadIdx.x], b = red[1][threadIdx.x], c = red[2][threadIdx.x],
               d = red[3][threadIdx.x];
  const int k = (4 * f) / C, col = (4 * f) % C;
  float *dst = k == 0 ? dg : (k == 1 ? db : dsum);
  if (!dst) return;
  unsafeAtomicAdd(&dst[col + 0], (a.x + b.x) + (c.x + d.x));
  unsafeAtomicAdd(&dst[col + 1], (a.y + b.y) + (c.y + d.y));
  unsafeAtomicAdd(&dst[col + 2], (a.z + b.z) + (c.z + d.z));
  unsafeAtomicAdd(&dst[col + 3], (a.w + b.w) + (c.w + d.w));
}

__global__ void __launch_bounds__(256) layernorm_bwd_reduce_kernel(int G, int C,
                                                                   const float *__restrict__ part,
                                                                   float *dg, float *db,
                                                                   float *dsum) {
  ln_reduce_body(G, C, part, dg, db, dsum);
}

// The same for several LayerNorm backward calls at once (one table entry per
// call, blockIdx.z): the whole-model step defers its 2L+1 reductions to one
// launch after the backward.
__global__ void __launch_bounds__(256) layernorm_bwd_reduce_batch_kernel(
    int G, int C, const LnReduceEntry *__restrict__ table) {
  const LnReduceEntry e = table[blockIdx.z];
  ln_reduce_body(G, C, e.part, e.dg, e.db, e.dsum);
}

// Vectorised column sums: each thread owns 16 bytes of a row (8 bf16 or 4
// f32 columns) and walks CS_ROWS rows of the workgroup's row slice in one of
// 8 row groups; LDS combines the groups, then one atomic per column.  Needs
// 16-byte aligned rows (host-checked).
constexpr int CS_ROWS = 128;   // rows per workgroup

template <bool BF16, bool F16 = false>
__global__ void __launch_bounds__(256) colsum_vec_kernel(int M, int N, int ld,
                                                         const void *__restrict__ src,
                                                         float *__restrict__ out) {
  constexpr int VEC = BF16 ? 8 : 4;
  const int ct = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int c0 = (blockIdx.x * 32 + ct) * VEC;
  const int m0 = blockIdx.y * CS_ROWS;
  const int m1 = min(M, m0 + CS_ROWS);
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  if (c0 < N) {
#pragma unroll 4
    for (int m = m0 + grp; m < m1; m += 8) {
      if (BF16) {
        const uint4 u = *(const uint4 *)((const bf16_t *)src + (size_t)m * ld + c0);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += lp_lo<F16>(w[q]);
          acc[2 * q + 1] += lp_hi<F16>(w[q]);
        }
      } else {
        const float4 f = *(const float4 *)((const float *)src + (size_t)m * ld + c0);
        acc[0] += f.x; acc[1] += f.y; acc[2] += f.z; acc[3] += f.w;
      }
    }
  }
  __shared__ float red[8][32 * VEC + 1];
#pragma unroll
  for (int i = 0; i < VEC; ++i) red[grp][ct * VEC + i] = acc[i];
  __syncthreads();
  const int c = blockIdx.x * 32 * VEC + threadIdx.x;
  if (threadIdx.x < 32 * VEC && c < N) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g) t += red[g][threadIdx.x];
    unsafeAtomicAdd(&out[c], t);
  }
}

// Column sums out[n] += sum_m src[m, n] (bias gradients).  Each block sums a
// strip of 64 columns over a slice of rows, then one atomic per column.
template <bool BF16, bool F16 = false>
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
      s += BF16 ? lp_to<F16>(((const bf16_t *)src)[(size_t)m * ld + col])
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
template <bool BF16, bool F16 = false>
__global__ void __launch_bounds__(256) ce_kernel(int N, int V, int ld, void *logits,
                                                 const int32_t *__restrict__ targets,
                                                 float *__restrict__ row_loss, float scale,
                                                 const float *__restrict__ scale_dev,
                                                 int32_t *flags) {
  if (scale_dev) scale *= *scale_dev;
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
        v[2 * q] = lp_lo<F16>(w[q]);
        v[2 * q + 1] = lp_hi<F16>(w[q]);
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
      float v = lp_to<F16>(z[i]);
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
      zy = y_ok ? lp_to<F16>(((const bf16_t *)logits)[(size_t)row * ld + y]) : NAN;
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
        float v0 = lp_lo<F16>(w[q]), v1 = lp_hi<F16>(w[q]);
        float d0 = c0 < V ? (__expf(v0 - lse) - (c0 == y ? 1.f : 0.f)) * scale : 0.f;
        float d1 = c1 < V ? (__expf(v1 - lse) - (c1 == y ? 1.f : 0.f)) * scale : 0.f;
        o[q] = lp_pack2<F16>(d0, d1);
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

// One-pass cross-entropy for bf16 rows of up to CE_VPT * 8 * 1024 columns: a
// 1024-thread workgroup holds its row in registers (CE_VPT 16-byte vectors per
// thread, branch-free buffer loads: vectors past the row read zero), reduces
// (max, sum exp) over the workgroup, then overwrites the row with
// (softmax - onehot) * scale; pad columns (>= V) become 0.  One read and one
// write of the logits instead of two reads and a write.
// Two workgroups share a CU (8 waves per SIMD, at most 64 VGPRs), so one
// row's reductions and stores overlap another's loads.  That fits only if
// the three passes each re-derive their unpacked values and indexes from the
// packed row: between passes the row and the thread index go through
// ce_opaque, which the compiler cannot see through (left alone it keeps 56
// unpacked floats and 7 store offsets live across the passes: 105 VGPRs, one
// workgroup per CU).
constexpr int CE_VPT = 7;
constexpr int CE_THREADS = 1024;

// An empty asm statement that claims to change x: values computed from the
// old x are not reused after it.  It emits no instruction.
__device__ __forceinline__ void ce_opaque(int &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void ce_opaque(uint4 &x) {
  asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
}

__device__ __forceinline__ float ce_block_reduce(float v, bool is_max, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < CE_THREADS / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
  __syncthreads();
  return r;
}

template <bool F16>
__global__ void __launch_bounds__(CE_THREADS, 8) ce_reg_kernel(int N, int V, int ld, bf16_t *logits,
                                                            const int32_t *__restrict__ targets,
                                                            float *__restrict__ row_loss,
                                                            float scale,
                                                            const float *__restrict__ scale_dev,
                                                            int32_t *flags) {
  if (scale_dev) scale *= *scale_dev;
  __shared__ float red[CE_THREADS / 64];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int y = targets[row];
  const bool y_ok = (y >= 0 && y < V);
  bf16_t *z = logits + (size_t)row * ld;
  const int nv8 = ld >> 3;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)z, (short)0, ld * 2, 0x00020000);
  uint4 v[CE_VPT];
#pragma unroll
  for (int i = 0; i < CE_VPT; ++i) {
    const int idx = tid + i * CE_THREADS;
    v[i] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, idx < nv8 ? (uint32_t)idx * 16u : 0x7ffffff0u,
                                                     0, 0));
  }
  const float zy = (tid == 0 && y_ok) ? lp_to<F16>(z[y]) : 0.f;   // read before any thread writes
  auto val = [&](int i, int q) {
    const uint32_t w = (&v[i].x)[q >> 1];
    return (q & 1) ? lp_hi<F16>(w) : lp_lo<F16>(w);
  };
  int tq = tid;
  ce_opaque(tq);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < CE_VPT; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if ((tq + i * CE_THREADS) * 8 + q < V) m = fmaxf(m, val(i, q));
  const float gm = ce_block_reduce(m, true, red);
#pragma unroll
  for (int i = 0; i < CE_VPT; ++i) ce_opaque(v[i]);
  ce_opaque(tq);
  float sacc = 0.f;
#pragma unroll
  for (int i = 0; i < CE_VPT; ++i)
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if ((tq + i * CE_THREADS) * 8 + q < V) sacc += __expf(val(i, q) - gm);
  const float lse = gm + __logf(ce_block_reduce(sacc, false, red));
#pragma unroll
  for (int i = 0; i < CE_VPT; ++i) ce_opaque(v[i]);
  ce_opaque(tq);
#pragma unroll
  for (int i = 0; i < CE_VPT; ++i) {
    const int idx = tq + i * CE_THREADS;
    if (idx >= nv8) continue;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c0 = idx * 8 + 2 * q, c1 = c0 + 1;
      const float d0 = c0 < V ? (__expf(val(i, 2 * q) - lse) - (c0 == y ? 1.f : 0.f)) * scale : 0.f;
      const float d1 = c1 < V ? (__expf(val(i, 2 * q + 1) - lse) - (c1 == y ? 1.f : 0.f)) * scale : 0.f;
      o[q] = lp_pack2<F16>(d0, d1);
    }
    ((uint4 *)z)[idx] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (tid == 0) {
    row_loss[row] = y_ok ? lse - zy : NAN;
    if (!y_ok) atomicOr(flags, 1);
  }
}

// Deterministic mean of n floats in one block.
// Mean of n values by one workgroup of 1024 threads, in a fixed order (the
// same bits every run): each thread sums a strided share with 8 independent
// loads in flight per round, then waves and workgroup reduce.
__global__ void __launch_bounds__(1024) mean_kernel(int n, const float *__restrict__ src,
                                                    float *__restrict__ out) {
  constexpr int U = 8;
  float s = 0.f;
  for (int i0 = threadIdx.x; i0 < n; i0 += 1024 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * 1024;
      v[u] = i < n ? src[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u];
  }
  __shared__ float red[16];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += red[w];
    out[0] = t / (float)n;
  }
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
                     (double)N * C * (4.0 + (tt_lowp(mode) ? 2.0 : 4.0)) + 8.0 * C + 8.0 * N);
#define TT_LNF(NV)                                                                              \
  if (nv <= NV) {                                                                               \
    if (mode == TT_BF16)                                                                        \
      hipLaunchKernelGGL((layernorm_fwd_kernel<true, NV>), grid, dim3(256), 0, ctx->stream, N, C, \
                         eps, x, g, b, y, mean, rstd);                                          \
    else if (mode == TT_FP16)                                                                   \
      hipLaunchKernelGGL((layernorm_fwd_kernel<true, NV, true>), grid, dim3(256), 0, ctx->stream, \
                         N, C, eps, x, g, b, y, mean, rstd);                                    \
    else                                                                                        \
      hipLaunchKernelGGL((layernorm_fwd_kernel<false, NV>), grid, dim3(256), 0, ctx->stream, N,   \
                         C, eps, x, g, b, y, mean, rstd);                                       \
    return tt_check_launch(ctx, "layernorm_fwd");                                               \
  }
  TT_LNF(1) TT_LNF(2) TT_LNF(3) TT_LNF(4) TT_LNF(8) TT_LNF(16)
#undef TT_LNF
  return TT_EUNSUPPORTED;
}

int tt_layernorm_bwd_groups(int N, int C) {
  const int nv = (C / 4 + 63) / 64;
  if (nv <= 4) {   // the row-walking kernel: 4 waves x lnp_rpw(N) rows per workgroup
    const int R = LNP_WAVES * lnp_rpw(N);
    return (N + R - 1) / R;
  }
  // the dispatched template width: the smallest of 8, 16 >= nv
  const int nvt = nv <= 8 ? 8 : 16;
  const int rows_per_wg = lnb_waves(nvt) * lnb_rpw(nvt);
  return (N + rows_per_wg - 1) / rows_per_wg;
}

// The group count is not monotone in N (the rows per wave of the row-walking
// kernel step from 2 to 4 to 8, which halves the count at each step), so a
// buffer for every N up to N_max takes the largest count over the regimes:
// within one regime the count grows with N, so the candidates are N_max and
// the regime ends below it.
int tt_layernorm_bwd_groups_max(int N_max, int C) {
  if (N_max <= 0) return 0;
  int G = tt_layernorm_bwd_groups(N_max, C);
  for (int r : {2, 4}) {
    const int end = LNP_MAX_WG * LNP_WAVES * r;   // last N with lnp_rpw(N) == r
    if (end < N_max) G = std::max(G, tt_layernorm_bwd_groups(end, C));
  }
  return G;
}

extern "C" int tt_layernorm_bwd_workspace(int n_rows, int C, size_t *bytes) {
  if (!bytes || n_rows < 0 || C <= 0 || C % 4 != 0 || C > 4096) return TT_EINVAL;
  *bytes = (size_t)tt_layernorm_bwd_groups_max(n_rows, C) * 3 * C * sizeof(float);
  return TT_OK;
}

int tt_layernorm_bwd_rows(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                          const float *mean, const float *rstd, const float *g, const float *dy,
                          const float *dres, float *dx, bf16_t *dx_bf16, float *part,
                          int part_groups) {
  TT_REQUIRE(ctx, N >= 0 && C > 0 && C % 4 == 0 && C <= 4096, "layernorm: need C %% 4 == 0, C <= 4096");
  TT_REQUIRE(ctx, x && mean && rstd && g && dy && dx && part, "layernorm_bwd: NULL pointer");
  if (N == 0) return TT_OK;
  const int nv = (C / 4 + 63) / 64;
  const int G = tt_layernorm_bwd_groups(N, C);
  TT_REQUIRE(ctx, G <= part_groups,
             "layernorm_bwd: %d rows need %d workgroup partials, the buffer holds %d", N, G,
             part_groups);
  const int rpw = lnp_rpw(N);   // rows per wave of the row-walking kernel (nv <= 4)
  {
    tt_prof_scope prof(ctx, nv <= 4 ? "layernorm_bwd_pipe_kernel" : "layernorm_bwd_kernel", 0.0,
                       (double)N * C * (12.0 + (dres ? 4.0 : 0.0) + (dx_bf16 ? 2.0 : 0.0)) +
                           8.0 * N + 12.0 * G * C);
#define TT_LNP_RPW(NV, RPW)                                                               \
      if (rpw == RPW) {                                                                   \
        if (mode == TT_FP16)                                                              \
          hipLaunchKernelGGL((layernorm_bwd_pipe_kernel<NV, RPW, true>), dim3(G),         \
                             dim3(64 * LNP_WAVES), 0, ctx->stream, N, C, x, mean, rstd, g, dy, \
                             dres, dx, dx_bf16, (float *)part);                           \
        else                                                                              \
          hipLaunchKernelGGL((layernorm_bwd_pipe_kernel<NV, RPW>), dim3(G),               \
                             dim3(64 * LNP_WAVES), 0, ctx->stream, N, C, x, mean, rstd, g, dy, \
                             dres, dx, dx_bf16, (float *)part);                           \
      } else
#define TT_LNP(NV)                                                                        \
    if (nv <= NV) {                                                                       \
      TT_LNP_RPW(NV, 2) TT_LNP_RPW(NV, 4) TT_LNP_RPW(NV, 8) return TT_EUNSUPPORTED;       \
    } else
#define TT_LNB(NV)                                                                        \
    if (nv <= NV) {                                                                       \
      if (mode == TT_FP16)                                                              \
        hipLaunchKernelGGL((layernorm_bwd_kernel<NV, true>), dim3(G), dim3(64 * lnb_waves(NV)), \
                           0, ctx->stream, N, C, x, mean, rstd, g, dy, dres, dx, dx_bf16, \
                           (float *)part);                                                \
      else                                                                                \
        hipLaunchKernelGGL((layernorm_bwd_kernel<NV>), dim3(G), dim3(64 * lnb_waves(NV)), 0, \
                           ctx->stream, N, C, x, mean, rstd, g, dy, dres, dx, dx_bf16,    \
                           (float *)part);                                                \
    } else
    TT_LNP(1) TT_LNP(2) TT_LNP(3) TT_LNP(4) TT_LNB(8) TT_LNB(16) return TT_EUNSUPPORTED;
#undef TT_LNP
#undef TT_LNP_RPW
#undef TT_LNB
  }
  return tt_check_launch(ctx, "layernorm_bwd");
}

int tt_layernorm_bwd_impl(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                          const float *mean, const float *rstd, const float *g, const float *dy,
                          const float *dres, float *dx, bf16_t *dx_bf16, float *dg, float *db,
                          float *dsum) {
  TT_REQUIRE(ctx, N >= 0 && C > 0 && C % 4 == 0 && C <= 4096, "layernorm: need C %% 4 == 0, C <= 4096");
  if (N == 0) return TT_OK;
  const int G = tt_layernorm_bwd_groups(N, C);
  tt_scratch_scope scope(ctx);
  void *part;
  TT_TRY(tt_arena_alloc(ctx, (size_t)G * 3 * C * 4, &part));
  return tt_layernorm_bwd_ws(ctx, mode, N, C, x, mean, rstd, g, dy, dres, dx, dx_bf16, dg, db,
                             dsum, (float *)part, G);
}

int tt_layernorm_bwd_ws(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                        const float *mean, const float *rstd, const float *g, const float *dy,
                        const float *dres, float *dx, bf16_t *dx_bf16, float *dg, float *db,
                        float *dsum, float *part, int part_groups) {
  TT_REQUIRE(ctx, N >= 0 && C > 0 && C % 4 == 0 && C <= 4096, "layernorm: need C %% 4 == 0, C <= 4096");
  if (N == 0) return TT_OK;
  const int G = tt_layernorm_bwd_groups(N, C);
  TT_TRY(tt_layernorm_bwd_rows(ctx, mode, N, C, x, mean, rstd, g, dy, dres, dx, dx_bf16, part,
                               part_groups));
  if (!dg && !db && !dsum) return TT_OK;
  tt_prof_scope prof(ctx, "layernorm_bwd_reduce_kernel", 0.0, 12.0 * G * C + 24.0 * C);
  hipLaunchKernelGGL(layernorm_bwd_reduce_kernel,
                     dim3((3 * C / 4 + 63) / 64, (G + LNR_SLICE - 1) / LNR_SLICE), dim3(256), 0,
                     ctx->stream, G, C, (const float *)part, dg, db, dsum);
  return tt_check_launch(ctx, "layernorm_bwd_reduce");
}

int tt_layernorm_bwd_reduce_batch(tt_ctx *ctx, int N, int C, const LnReduceEntry *table, int n) {
  TT_REQUIRE(ctx, table && n > 0 && n < 65536 && C > 0 && C % 4 == 0,
             "layernorm_bwd_reduce_batch: bad arguments");
  if (N == 0) return TT_OK;
  const int G = tt_layernorm_bwd_groups(N, C);
  tt_prof_scope prof(ctx, "layernorm_bwd_reduce_batch_kernel", 0.0,
                     n * (12.0 * G * C + 24.0 * C));
  hipLaunchKernelGGL(layernorm_bwd_reduce_batch_kernel,
                     dim3((3 * C / 4 + 63) / 64, (G + LNR_SLICE - 1) / LNR_SLICE, n), dim3(256), 0,
                     ctx->stream, G, C, table);
  return tt_check_launch(ctx, "layernorm_bwd_reduce_batch");
}

int tt_colsum(tt_ctx *ctx, int fmt, int M, int N, int ld, const void *src, float *out) {
  if (M == 0 || N == 0) return TT_OK;
  const bool src_bf16 = tt_lowp(fmt), f16 = fmt == TT_FP16;
  tt_prof_scope prof(ctx, "colsum_kernel", 0.0, (double)M * N * (src_bf16 ? 2.0 : 4.0) + 4.0 * N);
  const int vec = src_bf16 ? 8 : 4;
  if (tt_aligned16(src) && N % vec == 0 && ld % vec == 0) {
    dim3 grid((N / vec + 31) / 32, (M + CS_ROWS - 1) / CS_ROWS);
    if (f16)
      hipLaunchKernelGGL((colsum_vec_kernel<true, true>), grid, dim3(256), 0, ctx->stream, M, N, ld,
                         src, out);
    else if (src_bf16)
      hipLaunchKernelGGL(colsum_vec_kernel<true>, grid, dim3(256), 0, ctx->stream, M, N, ld, src, out);
    else
      hipLaunchKernelGGL(colsum_vec_kernel<false>, grid, dim3(256), 0, ctx->stream, M, N, ld, src, out);
    return tt_check_launch(ctx, "colsum");
  }
  int colblocks = (N + 63) / 64;
  int rowsplit = 1;
  while (colblocks * rowsplit < 1024 && rowsplit * 64 < M) rowsplit *= 2;
  int rpb = (M + rowsplit - 1) / rowsplit;
  dim3 grid(colblocks, (M + rpb - 1) / rpb);
  if (f16)
    hipLaunchKernelGGL((colsum_kernel<true, true>), grid, dim3(256), 0, ctx->stream, M, N, ld, rpb,
                       src, out);
  else if (src_bf16)
    hipLaunchKernelGGL(colsum_kernel<true>, grid, dim3(256), 0, ctx->stream, M, N, ld, rpb, src, out);
  else
    hipLaunchKernelGGL(colsum_kernel<false>, grid, dim3(256), 0, ctx->stream, M, N, ld, rpb, src, out);
  return tt_check_launch(ctx, "colsum");
}

int tt_ce_impl(tt_ctx *ctx, tt_mode mode, int N, int V, int ld, void *logits,
               const int32_t *targets, float *per_row_loss, float *loss, float grad_scale,
               const float *scale_dev) {
  TT_REQUIRE(ctx, N > 0 && V > 0 && ld >= V, "ce: bad shape N=%d V=%d ld=%d", N, V, ld);
  TT_REQUIRE(ctx, logits && targets && per_row_loss && loss, "ce: NULL pointer");
  {
  // algorithmic: one read and one write of the logits
  // (named after the kernel the row length selects)
  const bool reg = tt_lowp(mode) && ld <= CE_VPT * 8 * CE_THREADS;
  tt_prof_scope prof(ctx, reg ? "ce_reg_kernel" : "ce_kernel", 0.0,
                     2.0 * N * (double)ld * (tt_lowp(mode) ? 2.0 : 4.0) + 8.0 * N);
  if (tt_lowp(mode)) {
    TT_REQUIRE(ctx, ld % 8 == 0 && tt_aligned16(logits), "ce(16-bit): ld %% 8 and 16-byte alignment required");
    const bool f16 = mode == TT_FP16;
    if (reg) {
      if (f16)
        hipLaunchKernelGGL(ce_reg_kernel<true>, dim3(N), dim3(CE_THREADS), 0, ctx->stream, N, V, ld,
                           (bf16_t *)logits, targets, per_row_loss, grad_scale, scale_dev,
                           ctx->dev_flags);
      else
        hipLaunchKernelGGL(ce_reg_kernel<false>, dim3(N), dim3(CE_THREADS), 0, ctx->stream, N, V, ld,
                           (bf16_t *)logits, targets, per_row_loss, grad_scale, scale_dev,
                           ctx->dev_flags);
    } else if (f16) {
      hipLaunchKernelGGL((ce_kernel<true, true>), dim3(N), dim3(256), 0, ctx->stream, N, V, ld,
                         logits, targets, per_row_loss, grad_scale, scale_dev, ctx->dev_flags);
    } else {
      hipLaunchKernelGGL(ce_kernel<true>, dim3(N), dim3(256), 0, ctx->stream, N, V, ld, logits,
                         targets, per_row_loss, grad_scale, scale_dev, ctx->dev_flags);
    }
  } else {
    hipLaunchKernelGGL(ce_kernel<false>, dim3(N), dim3(256), 0, ctx->stream, N, V, ld, logits,
                       targets, per_row_loss, grad_scale, scale_dev, ctx->dev_flags);
  }
  }
  TT_TRY(tt_check_launch(ctx, "ce"));
  tt_prof_scope prof(ctx, "mean_kernel", 0.0, 4.0 * N);
  hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, ctx->stream, N, per_row_loss, loss);
  return tt_check_launch(ctx, "ce_mean");
}
