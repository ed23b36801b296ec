// bf16 MFMA GEMM for gfx950 (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// C[m,n] = sum_k A(m,k) B(k,n): the linear layer's forward and its two
// backward products (tinytorch page, §3 item 3).  Both operands are copied to
// LDS in their natural global layout with 16-byte loads, double-buffered.
// An MFMA lane needs 8 consecutive k values of one row of A / column of B:
//  * if the operand is k-contiguous ("k-major") the fragment is one 16-byte
//    LDS read;
//  * otherwise (the weight-gradient products reduce over the token index,
//    which is the row index of both operands) the fragment is assembled with
//    two ds_read_b64_tr_b16: within each 16-lane group, lane s points at 4
//    consecutive elements of row k0 + s/4, columns c0 + 4(s%4) .. +3, and
//    lane j then receives column c0 + j of rows k0 .. k0+3.
// Tile BM x BN x 64 per workgroup, WM x WN waves each owning a
// (BM/WM) x (BN/WN) block of 16x16 accumulator tiles.
#include <stdio.h>

#include <algorithm>
#include <vector>

#include "gemm_common.h"

namespace {

using namespace tt_gemm_detail;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int BK = 64;
constexpr int KPAD = 8;    // k-major rows: 72 elements (144 B) apart
constexpr int RPAD = 16;   // row-major rows: ROWS + 16 elements (shift of 32 B per row)
constexpr uint32_t OOB = 0x7ffffff0u;  // buffer offset past every operand (host: extent < 2 GB)

template <int ROWS, bool KM>
struct Operand {
  static constexpr int LD = KM ? (BK + KPAD) : (ROWS + RPAD);
  static constexpr int ELEMS = KM ? ROWS * LD : BK * LD;
  static constexpr int UNITS = ROWS * BK / 8;     // 16-byte vectors per tile

  // Global -> registers with buffer loads: the hardware returns zeros for
  // offsets at or past num_records, so an out-of-range vector is given the
  // offset OOB and no branch is needed.  Unit u covers 8 consecutive elements
  // along the contiguous dimension; consecutive lanes take consecutive units.
  // Rows past the matrix (m >= M, n >= N) only feed outputs that are not
  // stored; k >= K must read zero in at least one operand and never reach
  // another row's data, which the host guarantees (K % 8 == 0 whenever an
  // operand is k-major; row-major operands mask their k rows).
  template <int NT>
  __device__ __forceinline__ static void load(uint4 *reg, __amdgpu_buffer_rsrc_t rs, int ld, int r0,
                                              int k0, int R, int K, int tid) {
#pragma unroll
    for (int i = 0; i < UNITS / NT; ++i) {
      const int u = tid + i * NT;
      uint32_t off;
      if constexpr (KM) {
        const int r = r0 + u / (BK / 8), k = k0 + (u % (BK / 8)) * 8;
        off = (r < R && k < K) ? (uint32_t)(((size_t)r * ld + k) * 2) : OOB;
      } else {
        const int k = k0 + u / (ROWS / 8), r = r0 + (u % (ROWS / 8)) * 8;
        off = (k < K && r < R) ? (uint32_t)(((size_t)k * ld + r) * 2) : OOB;
      }
      reg[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
  }

  template <int NT>
  __device__ __forceinline__ static void store(bf16_t *s, const uint4 *reg, int tid) {
#pragma unroll
    for (int i = 0; i < UNITS / NT; ++i) {
      const int u = tid + i * NT;
      if constexpr (KM) {
        const int r = u / (BK / 8), k = (u % (BK / 8)) * 8;
        *(uint4 *)(s + r * LD + k) = reg[i];
      } else {
        const int k = u / (ROWS / 8), r = (u % (ROWS / 8)) * 8;
        *(uint4 *)(s + k * LD + r) = reg[i];
      }
    }
  }

  // MFMA fragment: rows rb .. rb+15 (lane%16), k = kk + 8*(lane/16) .. +7.
  __device__ __forceinline__ static bf16x8_t frag(const bf16_t *s, int rb, int kk, int lr, int lg) {
    if constexpr (KM) {
      return *(const bf16x8_t *)(s + (rb + lr) * LD + kk + 8 * lg);
    } else {
      const int kr = kk + 8 * lg + (lr >> 2);
      const int c = rb + 4 * (lr & 3);
      v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(s + kr * LD + c));
      v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(s + (kr + 4) * LD + c));
      typedef short v8s __attribute__((ext_vector_type(8)));
      v8s r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8_t, r);
    }
  }
};

template <int BM, int BN, int WM, int WN, bool A_KM, bool B_KM>
struct Cfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  using OA = Operand<BM, A_KM>;
  using OB = Operand<BN, B_KM>;
  static constexpr int STAGE = OA::ELEMS + OB::ELEMS;            // bf16 elements
  static constexpr int OPER_BYTES = 2 * STAGE * 2;
  static constexpr int LDC = BN + 4;
  static constexpr int EPI_BYTES = WTM * LDC * 4;                 // one wave-row of C, fp32
  static constexpr int SMEM = OPER_BYTES > EPI_BYTES ? OPER_BYTES : EPI_BYTES;
  static_assert(OA::UNITS % NT == 0 && OB::UNITS % NT == 0, "tile not divisible by threads");
  static_assert(SMEM <= 160 * 1024, "LDS");
};

// Occupancy target: two waves per SIMD (two 4-wave or one 8-wave workgroup
// per CU, capping registers at 256 per lane), except the 256x256 tile whose
// four waves each hold a 128x128 accumulator (one wave per SIMD).
template <int BM, int BN, int WM, int WN, bool A_KM, bool B_KM, bool F16 = false>
__global__ void __launch_bounds__(64 * WM * WN, (WM * WN == 4 && BM * BN < 256 * 256) ? 2 : 1)
gemm_bf16_kernel(GemmParams p) {
  using C = Cfg<BM, BN, WM, WN, A_KM, B_KM>;
  using OA = typename C::OA;
  using OB = typename C::OB;
  constexpr int NT = C::NT, FM = C::FM, FN = C::FN;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::SMEM];
  bf16_t *smem = (bf16_t *)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lg = lane >> 4;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.raster_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = blockIdx.z * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.B, (short)0, (int)p.b_bytes, 0x00020000);
  // Two register sets: the loads for stage it+2 are issued while stage it is
  // computed from LDS and stage it+1 waits in the other set.
  uint4 ra0[OA::UNITS / NT], rb0[OB::UNITS / NT], ra1[OA::UNITS / NT], rb1[OB::UNITS / NT];
  bf16_t *As[2] = {smem, smem + C::STAGE};
  bf16_t *Bs[2] = {smem + OA::ELEMS, smem + C::STAGE + OA::ELEMS};

  auto compute = [&](const bf16_t *as, const bf16_t *bs) {
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t fb[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = OB::frag(bs, wn * C::WTN + j * 16, kk, lr, lg);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        bf16x8_t fa = OA::frag(as, wm * C::WTM + i * 16, kk, lr, lg);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = lp_mfma<F16>(fa, fb[j], acc[i][j]);
      }
    }
  };

  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    OA::template load<NT>(ra0, rsa, p.lda, m0, kbeg, p.M, kend, tid);
    OB::template load<NT>(rb0, rsb, p.ldb, n0, kbeg, p.N, kend, tid);
    if (nk > 1) {
      OA::template load<NT>(ra1, rsa, p.lda, m0, kbeg + BK, p.M, kend, tid);
      OB::template load<NT>(rb1, rsb, p.ldb, n0, kbeg + BK, p.N, kend, tid);
    }
    OA::template store<NT>(As[0], ra0, tid);
    OB::template store<NT>(Bs[0], rb0, tid);
  }
  __syncthreads();
  for (int it = 0; it < nk; it += 2) {
    // even stage: compute buffer 0, set 0 is free -> stage it+2, store set 1 (stage it+1)
    if (it + 2 < nk) {
      OA::template load<NT>(ra0, rsa, p.lda, m0, kbeg + (it + 2) * BK, p.M, kend, tid);
      OB::template load<NT>(rb0, rsb, p.ldb, n0, kbeg + (it + 2) * BK, p.N, kend, tid);
    }
    compute(As[0], Bs[0]);
    if (it + 1 < nk) {
      OA::template store<NT>(As[1], ra1, tid);
      OB::template store<NT>(Bs[1], rb1, tid);
    }
    __syncthreads();
    if (it + 1 >= nk) break;
    // odd stage: compute buffer 1, set 1 is free -> stage it+3, store set 0 (stage it+2)
    if (it + 3 < nk) {
      OA::template load<NT>(ra1, rsa, p.lda, m0, kbeg + (it + 3) * BK, p.M, kend, tid);
      OB::template load<NT>(rb1, rsb, p.ldb, n0, kbeg + (it + 3) * BK, p.N, kend, tid);
    }
    compute(As[1], Bs[1]);
    if (it + 2 < nk) {
      OA::template store<NT>(As[0], ra0, tid);
      OB::template store<NT>(Bs[0], rb0, tid);
    }
    __syncthreads();
  }

  // Split-K partial sums go to their own slice of a workspace.
  if (p.out_zstride) p.out = (float *)p.out + blockIdx.z * p.out_zstride;
  // Epilogue, one wave-row of the tile at a time through LDS (fp32), then
  // row-coalesced 4-wide stores by all threads.
  float *Cs = (float *)smem_raw;
  constexpr int TPR = BN / 4, RPP = NT / TPR;
  const int cc = (tid % TPR) * 4;
  const int n = n0 + cc;
  const int nv = p.n_valid;
  float4 bias = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.bias && blockIdx.z == 0) {
    if (n + 3 < nv) {
      bias = *(const float4 *)(p.bias + n);
    } else {
      if (n < nv) bias.x = p.bias[n];
      if (n + 1 < nv) bias.y = p.bias[n + 1];
      if (n + 2 < nv) bias.z = p.bias[n + 2];
    }
  }
#pragma unroll
  for (int pass = 0; pass < WM; ++pass) {
    if (pass > 0) __syncthreads();
    if (wm == pass) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Cs[(i * 16 + lg * 4 + r) * C::LDC + wn * C::WTN + j * 16 + lr] = acc[i][j][r];
    }
    __syncthreads();
    for (int rr = tid / TPR; rr < C::WTM; rr += RPP) {
      const int m = m0 + pass * C::WTM + rr;
      if (m >= p.M || n >= nv) continue;
      float4 v = *(const float4 *)(Cs + rr * C::LDC + cc);
      v.x += bias.x; v.y += bias.y; v.z += bias.z; v.w += bias.w;
      epilogue4<F16>(p, m, n, v, nv - n);
    }
  }
}

template <int BM, int BN, int WM, int WN>
int launch(tt_ctx *ctx, const GemmArgs &g, int split, size_t out_zstride = 0) {
  GemmParams p{};
  p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.epi = g.epi; p.out = g.out; p.ldo = g.ldo; p.out_bf16 = g.out_bf16 ? 1 : 0;
  p.bias = g.bias; p.resid = g.resid; p.ldr = g.ldr; p.aux = g.aux; p.ldx = g.ldx;
  p.n_valid = g.n_valid > 0 ? min(g.n_valid, g.N) : g.N;
  p.vec_out = gemm_vec_out(g) ? 1 : 0;
  p.out_zstride = 0;
  p.raster_n = g.raster == 2 ? 1 : 0;
  p.a_bytes = (uint32_t)gemm_extent_bytes(g.a_kmajor, g.M, g.K, g.lda);
  p.b_bytes = (uint32_t)gemm_extent_bytes(g.b_kmajor, g.N, g.K, g.ldb);
  p.tiles_m = (g.M + BM - 1) / BM;
  p.tiles_n = (g.N + BN - 1) / BN;
  const int kb = (g.K + BK - 1) / BK;
  const int per = (kb + split - 1) / split;
  p.k_chunk = per * BK;
  split = (kb + per - 1) / per;
  p.out_zstride = out_zstride;
  dim3 grid(p.tiles_m * p.tiles_n, 1, split);
  const int li = (g.a_kmajor ? 2 : 0) + (g.b_kmajor ? 1 : 0);
  static char names[8][80];
  const int ni = li + (g.f16 ? 4 : 0);
  if (!names[ni][0])
    snprintf(names[ni], sizeof names[ni], "gemm_bf16_kernel<%d, %d, %d, %d, %s, %s, %s>", BM, BN, WM,
             WN, g.a_kmajor ? "true" : "false", g.b_kmajor ? "true" : "false",
             g.f16 ? "true" : "false");
  tt_prof_scope prof(ctx, names[ni], 2.0 * g.M * g.N * g.K, gemm_bytes(g));
#define TT_L(AK, BKM, H)                                                                       \
  if (g.a_kmajor == AK && g.b_kmajor == BKM && g.f16 == H) {                                   \
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, AK, BKM, H>), grid, dim3(64 * WM * WN), \
                       0, ctx->stream, p);                                                     \
    return tt_check_launch(ctx, "gemm_bf16");                                                  \
  }
  TT_L(true, true, false) TT_L(true, false, false) TT_L(false, true, false) TT_L(false, false, false)
  TT_L(true, true, true) TT_L(true, false, true) TT_L(false, true, true) TT_L(false, false, true)
#undef TT_L
  return TT_EINVAL;
}


// --------------------------------------------------------------------------
// v3: direct-to-LDS loads (buffer_load ... lds: lane i of a wave writes the
// 16 bytes it fetched at LDS base + 16 i), so no staging registers; an
// NSTAGE-deep ring of LDS tiles; one barrier per stage.  Tiles are unpadded
// and their 16-byte chunks XOR-swizzled so that the 16 lanes of one MFMA
// fragment read land on distinct banks:
//   k-major rows (BK elements):   physical chunk = chunk ^ swz_k(row)
//   row-major rows (ROWS elems):  physical chunk = chunk ^ rswz(k)
// (rswz spreads the rows k..k+3 and k+8..k+11 that two lane groups read in
// the same LDS cycle over 8 distinct chunk pairs).
// Each loading lane owns a fixed LDS slot and fetches the global chunk that
// belongs there.
// --------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

template <int ROWS, int BKV, bool KM>
struct DOp {
  static constexpr int ELEMS = ROWS * BKV;            // bf16 per stage
  static constexpr int BYTES = ELEMS * 2;
  static constexpr int CHUNKS = BYTES / 1024;         // 1 KB per wave instruction
  static constexpr int CPR = KM ? BKV / 8 : ROWS / 8; // 16-byte chunks per LDS row
  static constexpr int RB = KM ? BKV * 2 : ROWS * 2;  // bytes per LDS row
  static_assert(BYTES % 1024 == 0, "tile must be whole 1 KB wave loads");
  // The XOR swizzles stay inside a row only for power-of-two chunk counts, and
  // the row-major one flips chunk bits up to 8 (needs >= 16 chunks per row).
  static constexpr bool VALID =
      (CPR & (CPR - 1)) == 0 && (KM || CPR >= 16);

  // chunk swizzle of k-major row r: rows are paired (measured: pairing gives
  // fewer LDS bank conflicts than one swizzle value per 256 bytes of rows
  // for 64-byte rows, and is the same thing for 128-byte rows)
  __device__ __forceinline__ static int swz_k(int r) { return (r >> 1) % CPR; }
  __device__ __forceinline__ static int rswz(int k) { return 2 * ((k & 3) | ((k >> 1) & 4)); }

  // Issue this wave's share of the tile's loads (chunk instructions w, w+NW,
  // ...).  When the chunks do not divide evenly, the first CHUNKS % NW waves
  // issue one more (the count stays uniform within a wave).
  template <int NW>
  __device__ __forceinline__ static void issue(bf16_t *tile, __amdgpu_buffer_rsrc_t rs, int ld,
                                               int r0, int k0, int R, int K, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < (CHUNKS + NW - 1) / NW; ++i) {
      const int ci = wave + i * NW;
      if (CHUNKS % NW != 0 && ci >= CHUNKS) break;
      const int L = ci * 64 + lane;            // linear 16-byte slot in the tile
      uint32_t off;
      if constexpr (KM) {
        const int r = L / CPR, pc = L % CPR;
        const int lc = pc ^ swz_k(r);
        const int gr = r0 + r, gk = k0 + lc * 8;
        off = (gr < R && gk < K) ? (uint32_t)(((size_t)gr * ld + gk) * 2) : OOB;
      } else {
        const int k = L / CPR, pc = L % CPR;
        const int lc = pc ^ rswz(k);
        const int gk = k0 + k, gr = r0 + lc * 8;
        off = (gk < K && gr < R) ? (uint32_t)(((size_t)gk * ld + gr) * 2) : OOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)((char *)tile + ci * 1024), 16, off,
                                               0, 0, 0);
    }
  }

  // Fragment: rows rb + lane%16, k = kk + 8 (lane/16) .. +7.
  __device__ __forceinline__ static bf16x8_t frag(const bf16_t *t, int rb, int kk, int lr, int lg) {
    if constexpr (KM) {
      const int r = rb + lr;
      const int pc = ((kk >> 3) + lg) ^ swz_k(r);
      return *(const bf16x8_t *)(t + r * BKV + pc * 8);
    } else {
      const int c = rb + 4 * (lr & 3);
      const int kr0 = kk + 8 * lg + (lr >> 2);
      const int kr1 = kr0 + 4;
      const int pc0 = (c >> 3) ^ rswz(kr0), pc1 = (c >> 3) ^ rswz(kr1);
      v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(t + kr0 * ROWS + pc0 * 8 + (c & 7)));
      v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(t + kr1 * ROWS + pc1 * 8 + (c & 7)));
      typedef short v8s __attribute__((ext_vector_type(8)));
      v8s v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // Row-major operand: LDS byte address of the first of a fragment's two
  // transpose reads.  The second is TR_STEP bytes further: its rows are 4
  // further (k0 + 4 .. k0 + 7 with k0 % 8 < 4, so rswz and the swizzled
  // chunk are the same).
  static constexpr int TR_STEP = 4 * ROWS * 2;
  __device__ __forceinline__ static uint32_t tr_addr(const bf16_t *t, int rb, int kk, int lr, int lg) {
    const int c = rb + 4 * (lr & 3);
    const int kr0 = kk + 8 * lg + (lr >> 2);
    const int pc0 = (c >> 3) ^ rswz(kr0);
    return (uint32_t)(uintptr_t)(lds_v4s *)(t + kr0 * ROWS + pc0 * 8 + (c & 7));
  }
};

// The weight-gradient tile's fragments (256 x 128, 4 x 2 waves: four of A,
// four of B per 32-deep stage, both operands row-major): 16 transpose reads
// and their wait (lgkmcnt(0)) in ONE asm statement.  Through the builtin, the
// compiler puts a full vmcnt(0) wait in front of a transpose read whenever a
// buffer-to-LDS load is in flight (it cannot tell the ring's stages apart),
// which would drain the ring every stage; it does not look into inline
// assembly.  With the wait inside the statement, no fragment register can be
// read (or copied) before its data has landed.
__device__ __forceinline__ void tr_frags_4x4(const uint32_t (&aa)[4], const uint32_t (&ab)[4],
                                             bf16x8_t (&fa)[4], bf16x8_t (&fb)[4]) {
  v4s a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3, b4, b5, b6, b7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:1024\n\t"
      "ds_read_b64_tr_b16 %10, %21\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:1024\n\t"
      "ds_read_b64_tr_b16 %12, %22\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:1024\n\t"
      "ds_read_b64_tr_b16 %14, %23\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(a4), "=&v"(a5), "=&v"(a6), "=&v"(a7),
        "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3), "=&v"(b4), "=&v"(b5), "=&v"(b6), "=&v"(b7)
      : "v"(aa[0]), "v"(aa[1]), "v"(aa[2]), "v"(aa[3]), "v"(ab[0]), "v"(ab[1]), "v"(ab[2]),
        "v"(ab[3])
      : "memory");
  typedef short v8s __attribute__((ext_vector_type(8)));
  fa[0] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  fa[1] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(a2, a3, 0, 1, 2, 3, 4, 5, 6, 7));
  fa[2] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(a4, a5, 0, 1, 2, 3, 4, 5, 6, 7));
  fa[3] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(a6, a7, 0, 1, 2, 3, 4, 5, 6, 7));
  fb[0] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  fb[1] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(b2, b3, 0, 1, 2, 3, 4, 5, 6, 7));
  fb[2] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(b4, b5, 0, 1, 2, 3, 4, 5, 6, 7));
  fb[3] = __builtin_bit_cast(bf16x8_t, (v8s)__builtin_shufflevector(b6, b7, 0, 1, 2, 3, 4, 5, 6, 7));
}

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}


template <int BM, int BN, int BKV, int WM, int WN, int NS, bool A_KM, bool B_KM>
struct Cfg3 {
  static constexpr int BM_ = BM, BN_ = BN, WM_ = WM, WN_ = WN;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  using OA = DOp<BM, BKV, A_KM>;
  using OB = DOp<BN, BKV, B_KM>;
  static constexpr int STAGE = OA::ELEMS + OB::ELEMS;
  // Loads per stage of the wave with the fewest (waves may differ by one per
  // operand): the vmcnt waits count with it, which for the other waves waits
  // for at most one load of a later stage besides the stage needed.
  static constexpr int LPS = OA::CHUNKS / NW + OB::CHUNKS / NW;
  static constexpr int OPER_BYTES = NS * STAGE * 2;
  static constexpr int LDC = BN + 4;
  static constexpr int EPI_BYTES = WTM * LDC * 4;
  static constexpr int SMEM = OPER_BYTES > EPI_BYTES ? OPER_BYTES : EPI_BYTES;
  static_assert(SMEM <= 160 * 1024, "LDS");
  static_assert((NS - 2) * LPS < 64, "vmcnt range");
  // workgroups per CU that the LDS allows (at most 2), as waves per SIMD
  static constexpr int WG_PER_CU = 2 * SMEM <= 160 * 1024 ? 2 : 1;
  static constexpr int WAVES_PER_EU = (NW * WG_PER_CU + 3) / 4;
};

// A workgroup barrier for LDS reuse only: every wave's LDS accesses have
// completed (lgkmcnt(0)) before any wave passes.  Unlike __syncthreads() it
// does not wait for the wave's outstanding global stores -- between the
// epilogue's passes that wait costs a full store round trip per pass -- and
// the stores need no ordering among themselves.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum of column c over the first ROWS rows of a staged tile (row stride LD):
// four interleaved partial sums, added in a fixed order at the end, so the
// LDS reads are not one serial add chain.
template <int ROWS, int LD>
__device__ __forceinline__ float column_sum(const float *t, int c) {
  static_assert(ROWS % 4 == 0, "rows in fours");
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 4
  for (int r = 0; r < ROWS; r += 4) {
    s0 += t[r * LD + c];
    s1 += t[(r + 1) * LD + c];
    s2 += t[(r + 2) * LD + c];
    s3 += t[(r + 3) * LD + c];
  }
  return (s0 + s1) + (s2 + s3);
}

// Epilogue shared by the direct-to-LDS kernels: the C tile goes through LDS
// one wave-row at a time (fp32), then every thread applies the activation /
// residual to 4 consecutive columns with row-coalesced accesses; optional
// column sums of the stored values (bias gradients).  The bias is already in
// the accumulators (the kernels start them from it), so the row loops issue
// no loads of their own but the residual / pre-activation ones: a load in the
// loop would make every row wait for the stores of the rows before it.  The
// caller has passed a barrier after the last LDS read of the main loop.
template <class C, bool F16>
__device__ __forceinline__ void v3_epilogue(GemmParams &p, f32x4_t (&acc)[C::FM][C::FN], char *smem_raw,
                                            int m0, int n0) {
  constexpr int NT = C::NT, FM = C::FM, FN = C::FN, BN = C::BN_, WM = C::WM_, WN = C::WN_;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lg = lane >> 4;
  if (p.out_zstride) p.out = (float *)p.out + blockIdx.z * p.out_zstride;
  float *Cs = (float *)smem_raw;
  constexpr int TPR = BN / 4;
  if constexpr (NT % TPR != 0) {
    // Flattened epilogue (a thread's column group changes between rows).
    // Column sums: the stored values go back into the staged tile and
    // thread t < BN adds up column t after each pass.
    const int nv = p.n_valid;
    float csum = 0.f;
    // The GELU-backward product: every pre-activation load of this thread's
    // items, over all passes, is issued before the first pass stages its
    // rows -- one memory round trip for the tile instead of one per pass
    // (or per item).
    // (Only for wave tiles of at most 16 MFMA blocks: beside larger
    // accumulator sets the prefetch array would not fit the registers.)
    constexpr int ITEMS = (C::WTM * TPR + NT - 1) / NT;
    constexpr bool GB_PREFETCH = FM * FN <= 16;
    const bool gelu_bwd = GB_PREFETCH && p.epi == EPI_GELU_BWD && p.out_bf16 && p.vec_out;
    uint2 hv[GB_PREFETCH ? WM : 1][GB_PREFETCH ? ITEMS : 1];
    if constexpr (GB_PREFETCH) if (gelu_bwd) {
#pragma unroll
      for (int pass = 0; pass < WM; ++pass)
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
          const int idx = tid + it * NT;
          const int rr = idx / TPR, cc = (idx % TPR) * 4;
          const int m = m0 + pass * C::WTM + rr, n = n0 + cc;
          hv[pass][it] = make_uint2(0u, 0u);
          if (idx < C::WTM * TPR && m < p.M && n + 3 < nv)
            hv[pass][it] = *(const uint2 *)((const bf16_t *)p.aux + (size_t)m * p.ldx + n);
        }
    }
#pragma unroll
    for (int pass = 0; pass < WM; ++pass) {
      if (pass > 0) lds_barrier();
      if (wm == pass) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              Cs[(i * 16 + lg * 4 + r) * C::LDC + wn * C::WTN + j * 16 + lr] = acc[i][j][r];
      }
      lds_barrier();
      if constexpr (GB_PREFETCH) if (gelu_bwd) {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
          const int idx = tid + it * NT;
          if (idx >= C::WTM * TPR) break;
          const int rr = idx / TPR, cc = (idx % TPR) * 4;
          const int m = m0 + pass * C::WTM + rr, n = n0 + cc;
          float4 *cp = (float4 *)(Cs + rr * C::LDC + cc);
          if (m >= p.M || n >= nv) {
            if (p.colsum) *cp = make_float4(0.f, 0.f, 0.f, 0.f);
            continue;
          }
          const float4 v = *cp;
          float4 st;
          if (n + 3 < nv) {
            const uint2 hp = hv[pass][it];
            const float h[4] = {lp_lo<F16>(hp.x), lp_hi<F16>(hp.x), lp_lo<F16>(hp.y), lp_hi<F16>(hp.y)};
            const float a[4] = {v.x * gelu_grad_f(h[0]), v.y * gelu_grad_f(h[1]),
                                v.z * gelu_grad_f(h[2]), v.w * gelu_grad_f(h[3])};
            out_store((bf16_t *)p.out + (size_t)m * p.ldo + n,
                      make_uint2(lp_pack2<F16>(a[0], a[1]), lp_pack2<F16>(a[2], a[3])));
            st = round_stored<F16>(p, a, 4);
          } else {
            st = epilogue4<F16>(p, m, n, v, nv - n);   // the ragged last columns
          }
          if (p.colsum) *cp = st;
        }
        if (p.colsum) {
          lds_barrier();
          if (tid < BN) csum += column_sum<C::WTM, C::LDC>(Cs, tid);
        }
        continue;
      }
      for (int idx = tid; idx < C::WTM * TPR; idx += NT) {
        const int rr = idx / TPR, cc = (idx % TPR) * 4;
        const int m = m0 + pass * C::WTM + rr, n = n0 + cc;
        float4 *cp = (float4 *)(Cs + rr * C::LDC + cc);
        if (m >= p.M || n >= nv) {
          if (p.colsum) *cp = make_float4(0.f, 0.f, 0.f, 0.f);
          continue;
        }
        const float4 st = epilogue4<F16>(p, m, n, *cp, nv - n);
        if (p.colsum) *cp = st;
      }
      if (p.colsum) {
        lds_barrier();
        if (tid < BN) csum += column_sum<C::WTM, C::LDC>(Cs, tid);
      }
    }
    if (p.colsum && tid < BN && n0 + tid < nv) unsafeAtomicAdd(&p.colsum[n0 + tid], csum);
    return;
  }
  constexpr int RPP = NT / TPR;
  const int cc = (tid % TPR) * 4;
  const int n = n0 + cc;
  const int nv = p.n_valid;
  float4 csum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int pass = 0; pass < WM; ++pass) {
    if (pass > 0) lds_barrier();
    if (wm == pass) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Cs[(i * 16 + lg * 4 + r) * C::LDC + wn * C::WTN + j * 16 + lr] = acc[i][j][r];
    }
    lds_barrier();
    for (int rr = tid / TPR; rr < C::WTM; rr += RPP) {
      const int m = m0 + pass * C::WTM + rr;
      if (m >= p.M || n >= nv) continue;
      const float4 st = epilogue4<F16>(p, m, n, *(const float4 *)(Cs + rr * C::LDC + cc), nv - n);
      csum.x += st.x; csum.y += st.y; csum.z += st.z; csum.w += st.w;
    }
  }
  // Column sums of the stored tile (bias gradients): combine the RPP row
  // groups in LDS, then one atomic per column and workgroup.
  if (p.colsum) {
    lds_barrier();
    float *red = (float *)smem_raw;   // [RPP][BN]
    *(float4 *)&red[(tid / TPR) * BN + cc] = csum;
    lds_barrier();
    for (int c = tid; c < BN; c += NT) {
      float t = 0.f;
#pragma unroll
      for (int r = 0; r < RPP; ++r) t += red[r * BN + c];
      if (n0 + c < nv) unsafeAtomicAdd(&p.colsum[n0 + c], t);
    }
  }
}

template <int BM, int BN, int BKV, int WM, int WN, int NS, bool A_KM, bool B_KM, bool GROUP = false,
          bool F16 = false>
__global__ void __launch_bounds__(64 * WM * WN,
                                  (Cfg3<BM, BN, BKV, WM, WN, NS, A_KM, B_KM>::WAVES_PER_EU))
gemm_bf16_v3_kernel(GemmParams p) {
  using C = Cfg3<BM, BN, BKV, WM, WN, NS, A_KM, B_KM>;
  using OA = typename C::OA;
  using OB = typename C::OB;
  constexpr int NW = C::NW, NT = C::NT, FM = C::FM, FN = C::FN;
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::SMEM];
  bf16_t *smem = (bf16_t *)smem_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lg = lane >> 4;
  int tm, tn;
  if constexpr (GROUP) {
    // Grouped launch: spread the grid XCD-first (the grid is padded to a
    // multiple of 8), find the problem that owns this workgroup, and take its
    // operands, output and shape (the tile order inside a problem has no XCD
    // step of its own).
    const int nwg = gridDim.x;
    const int bid = (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8;
    const int e = p.group_map[bid];
    if (e == 0xffff) return;   // padding: the whole workgroup leaves
    const GemmGroupEntry q = p.group[e];
    p.A = q.A; p.B = q.B; p.out = q.out;
    p.lda = q.lda; p.ldb = q.ldb; p.ldo = q.ldo;
    p.M = q.M; p.N = q.N; p.n_valid = q.N;
    p.tiles_m = q.tiles_m; p.tiles_n = q.tiles_n; p.vec_out = q.vec_out;
    p.a_bytes = (uint32_t)gemm_extent_bytes(false, q.M, p.K, q.lda);
    p.b_bytes = (uint32_t)gemm_extent_bytes(false, q.N, p.K, q.ldb);
    tile_coords(bid - q.tile0, q.tiles_m * q.tiles_n, q.tiles_m, q.tiles_n, q.raster_n, tm, tn,
                false);
  } else {
    tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.raster_n, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = blockIdx.z * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.B, (short)0, (int)p.b_bytes, 0x00020000);

  // The bias starts the accumulators (lane columns wn WTN + 16 j + lane % 16;
  // only the first k split carries it).  Its loads go out ahead of the
  // operand prologue and land under it.
  float bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * C::WTN + j * 16 + lr;
    bcol[j] = !GROUP && p.bias && blockIdx.z == 0 && n < p.n_valid ? p.bias[n] : 0.f;
  }
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{bcol[j], bcol[j], bcol[j], bcol[j]};

  auto At = [&](int s) { return smem + s * C::STAGE; };
  auto Bt = [&](int s) { return smem + s * C::STAGE + OA::ELEMS; };
  auto issue = [&](int stage, int buf) {
    const int k0 = kbeg + stage * BKV;
    OA::template issue<NW>(At(buf), rsa, p.lda, m0, k0, p.M, kend, wave, lane);
    OB::template issue<NW>(Bt(buf), rsb, p.ldb, n0, k0, p.N, kend, wave, lane);
  };
  const int nk = (kend - kbeg + BKV - 1) / BKV;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s);
  {
    for (int it = 0; it < nk; ++it) {
      // Stage it must have landed (from every wave) before anyone reads it:
      // each wave waits for its own loads of that stage, then a bare barrier
      // (no memory fence, which would also drain the loads still in flight
      // for later stages).  The buffer refilled below was last read in
      // iteration it-1, whose LDS reads every wave has consumed before
      // reaching here.  The empty asm statements keep the compiler from
      // moving LDS accesses across the barrier (the barrier builtin is not a
      // memory operation to it); they emit no instruction and no wait.
      if (it + NS - 2 < nk) wait_vm<(NS - 2) * C::LPS>();
      else wait_vm<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const bf16_t *as = At(it % NS), *bs = Bt(it % NS);
      if constexpr (A_KM && B_KM) {
        if (it + NS - 1 < nk) issue(it + NS - 1, (it + NS - 1) % NS);
        // Every fragment of the stage is read into registers of its own; the
        // scheduling barriers then fix the order: the first k step's reads,
        // its MFMAs with the next step's reads spread between them, the
        // remaining MFMAs.  Left to itself the compiler reads each fragment
        // just before its first MFMA and waits for it there.
        constexpr int KS = BKV / 32;
        constexpr int RD = FM + FN;   // LDS reads per k step
        constexpr int MF = FM * FN;   // MFMAs per k step
        constexpr int PER = MF / RD > 0 ? MF / RD : 1;
        bf16x8_t fa[KS][FM], fb[KS][FN];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
          for (int j = 0; j < FN; ++j) fb[s][j] = OB::frag(bs, wn * C::WTN + j * 16, s * 32, lr, lg);
#pragma unroll
          for (int i = 0; i < FM; ++i) fa[s][i] = OA::frag(as, wm * C::WTM + i * 16, s * 32, lr, lg);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = lp_mfma<F16>(fa[s][i], fb[s][j], acc[i][j]);
        __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);       // DS reads
#pragma unroll
        for (int s = 1; s < KS; ++s) {
#pragma unroll
          for (int q = 0; q < RD; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);  // MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if constexpr (MF - PER * RD > 0) __builtin_amdgcn_sched_group_barrier(0x008, MF - PER * RD, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
      } else if constexpr (!A_KM && !B_KM && BM == 256 && BN == 128 && WM == 4 && WN == 2 &&
                           BKV == 32) {
        // The weight-gradient tile: next stage issued, then the stage's
        // transpose reads and their wait in one asm statement
        // (tr_frags_4x4), then the MFMAs while those loads are in flight.
        static_assert(FM == 4 && FN == 4 && OA::TR_STEP == 2048 && OB::TR_STEP == 1024,
                      "tr_frags_4x4 hard-codes this tile's fragment counts and read offsets");
        if (it + NS - 1 < nk) issue(it + NS - 1, (it + NS - 1) % NS);
        uint32_t aa[4], ab[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) aa[i] = OA::tr_addr(as, wm * C::WTM + i * 16, 0, lr, lg);
#pragma unroll
        for (int j = 0; j < 4; ++j) ab[j] = OB::tr_addr(bs, wn * C::WTN + j * 16, 0, lr, lg);
        bf16x8_t fa[4], fb[4];
        tr_frags_4x4(aa, ab, fa, fb);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = lp_mfma<F16>(fa[i], fb[j], acc[i][j]);
      } else {
        // Other tiles with a row-major operand (the builtin transpose read;
        // the compiler's vmcnt(0) in front of it then drains the ring, so
        // the next stage is issued after the reads): not on the step's path.
        constexpr int KS = BKV / 32;
        bf16x8_t fa[KS][FM], fb[KS][FN];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
          for (int j = 0; j < FN; ++j) fb[s][j] = OB::frag(bs, wn * C::WTN + j * 16, s * 32, lr, lg);
#pragma unroll
          for (int i = 0; i < FM; ++i) fa[s][i] = OA::frag(as, wm * C::WTM + i * 16, s * 32, lr, lg);
        }
        asm volatile("" ::: "memory");
        if (it + NS - 1 < nk) issue(it + NS - 1, (it + NS - 1) % NS);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = lp_mfma<F16>(fa[s][i], fb[s][j], acc[i][j]);
      }
    }
  }
  __syncthreads();
  v3_epilogue<C, F16>(p, acc, smem_raw, m0, n0);
}

template <int BM, int BN, int BKV, int WM, int WN, int NS>
int launch3(tt_ctx *ctx, const GemmArgs &g, int split, size_t out_zstride = 0) {
  GemmParams p{};
  p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.epi = g.epi; p.out = g.out; p.ldo = g.ldo; p.out_bf16 = g.out_bf16 ? 1 : 0;
  p.bias = g.bias; p.resid = g.resid; p.ldr = g.ldr; p.aux = g.aux; p.ldx = g.ldx;
  p.n_valid = g.n_valid > 0 ? min(g.n_valid, g.N) : g.N;
  p.vec_out = gemm_vec_out(g) ? 1 : 0;
  p.out_zstride = out_zstride;
  p.colsum = split == 1 ? g.colsum : nullptr;
  p.raster_n = g.raster == 2 ? 1 : 0;
  p.a_bytes = (uint32_t)gemm_extent_bytes(g.a_kmajor, g.M, g.K, g.lda);
  p.b_bytes = (uint32_t)gemm_extent_bytes(g.b_kmajor, g.N, g.K, g.ldb);
  p.tiles_m = (g.M + BM - 1) / BM;
  p.tiles_n = (g.N + BN - 1) / BN;
  const int kb = (g.K + BKV - 1) / BKV;
  const int per = (kb + split - 1) / split;
  p.k_chunk = per * BKV;
  split = (kb + per - 1) / per;
  dim3 grid(p.tiles_m * p.tiles_n, 1, split);
  static char names[8][112];
  const int li = (g.a_kmajor ? 2 : 0) + (g.b_kmajor ? 1 : 0) + (g.f16 ? 4 : 0);
  if (!names[li][0])
    snprintf(names[li], sizeof names[li],
             "gemm_bf16_v3_kernel<%d, %d, %d, %d, %d, %d, %s, %s, false, %s>", BM, BN, BKV, WM, WN,
             NS, g.a_kmajor ? "true" : "false", g.b_kmajor ? "true" : "false",
             g.f16 ? "true" : "false");
  tt_prof_scope prof(ctx, names[li], 2.0 * g.M * g.N * g.K, gemm_bytes(g));
#define TT_L3(AK, BKM, H)                                                                       \
  if (g.a_kmajor == AK && g.b_kmajor == BKM && g.f16 == H) {                                    \
    if constexpr (DOp<BM, BKV, AK>::VALID && DOp<BN, BKV, BKM>::VALID) {                        \
      hipLaunchKernelGGL((gemm_bf16_v3_kernel<BM, BN, BKV, WM, WN, NS, AK, BKM, false, H>), grid, \
                         dim3(64 * WM * WN), 0, ctx->stream, p);                                \
      return tt_check_launch(ctx, "gemm_bf16_v3");                                              \
    } else {                                                                                    \
      return tt_set_error(ctx, TT_EUNSUPPORTED, "gemm_bf16_v3: tile/layout not supported");    \
    }                                                                                           \
  }
  TT_L3(true, true, false) TT_L3(true, false, false) TT_L3(false, true, false)
  TT_L3(false, false, false) TT_L3(true, true, true) TT_L3(true, false, true)
  TT_L3(false, true, true) TT_L3(false, false, true)
#undef TT_L3
  return TT_EINVAL;
}

// --------------------------------------------------------------------------
// Ping-pong k-major GEMM (both operands k-major), used for the N = 768
// products of the step (attention and MLP down-projections, the dX of the
// qkv and fc layers, the LM-head dH).  One workgroup of 8 waves owns a
// 128 x BN output tile.  The waves form two groups of four -- waves 0-3 and
// 4-7, so every SIMD holds one wave of each -- and the groups take alternate
// BKP-deep k-stages (group 0 the even ones, group 1 the odd ones), each group
// with an LDS ring of its own NSG stages.  Each wave accumulates a 128 x
// (BN/4) block of its group's partial tile (8 x BN/64 MFMA tiles of 16 x 16),
// which keeps the LDS bytes read per MFMA low: (128 + BN/4) / (128 BN/4) per
// output element and k, about 0.6x those of a 64 x 48 block.  128 x 192
// tiles put exactly 256 workgroups on the N = 768 products (one per CU).
//
// The groups run in alternating phases, offset by one: while one group
// issues its MFMAs for a stage, the other reads its next stage's fragments
// from LDS and issues the global loads of a later stage into its ring.  Each
// phase ends with one workgroup barrier, so on every SIMD the MFMA wave and
// the memory wave of a phase run side by side, and the MFMA pipe always has
// a wave with a stage in registers.  Loads run D = NSG - 1 of a group's
// stages ahead; a wave waits for its own loads of the stage it reads next
// (vmcnt) before the barrier that opens that stage, and reads complete
// (lgkmcnt(0)) before the barrier that closes its memory phase, so a ring
// slot is refilled only after its readers are done with it.
//
// At the end the two partial tiles meet in LDS (group 0 stores, group 1
// adds: a fixed order, so the result is deterministic) and all 512 threads
// run the usual epilogue with row-coalesced accesses.
//
// Measured (single products, MI355X): with the global loads removed the
// schedule runs the LM-head dH at 1.67 PFLOP/s, so the MFMA/LDS side is not
// the limit; with them, the operand stream bounds it (1.05 PFLOP/s).  64-deep
// stages (whole 128-byte lines per k-major row) beat 32-deep ones by 5-25 %.
// --------------------------------------------------------------------------
template <int BN, int NSG, int BKP = 32>
struct PPCfg {
  static constexpr int BM = 128, BK = BKP, NW = 8, NT = 512, GW = 4;
  static constexpr int KS = BK / 32;               // MFMA k-steps per stage
  static constexpr int WTN = BN / GW;              // columns per wave
  static constexpr int FM = BM / 16, FN = WTN / 16;
  using OA = DOp<BM, BK, true>;
  using OB = DOp<BN, BK, true>;
  static constexpr int STAGE = OA::ELEMS + OB::ELEMS;   // bf16 elements
  static constexpr int LPW = OA::CHUNKS / GW + OB::CHUNKS / GW;   // loads per wave per stage
  static constexpr int RING = NSG * STAGE;                      // per group
  static constexpr int OPER_BYTES = 2 * RING * 2;
  static constexpr int LDC = BN + 4;
  static constexpr int EPI_BYTES = BM * LDC * 4;
  static constexpr int SMEM = OPER_BYTES > EPI_BYTES ? OPER_BYTES : EPI_BYTES;
  static_assert(WTN % 16 == 0, "BN must be a multiple of 64");
  static_assert(OA::CHUNKS % GW == 0 && OB::CHUNKS % GW == 0, "loads not divisible by waves");
  static_assert(SMEM <= 160 * 1024, "LDS");
  static_assert(NSG >= 2 && (NSG - 2) * LPW < 64, "ring depth / vmcnt range");
};

// s_waitcnt lgkmcnt(0), other counters left alone.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A workgroup barrier that nothing crosses: the empty asm statements keep
// memory accesses on their side at the IR level, the scheduling barriers keep
// every instruction (the MFMAs included) on its side in the machine
// scheduler.
__device__ __forceinline__ void pp_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// vmcnt(r * LPW) for r in [0, 3]: loads of the last r stages may still fly.
template <int LPW>
__device__ __forceinline__ void wait_vm_stages(int r) {
  if (r >= 3) wait_vm<3 * LPW>();
  else if (r == 2) wait_vm<2 * LPW>();
  else if (r == 1) wait_vm<LPW>();
  else wait_vm<0>();
}

template <int BN, int NSG, int BKP, bool F16>
__global__ void __launch_bounds__(512, 1) gemm_pp_kernel(GemmParams p) {
  using C = PPCfg<BN, NSG, BKP>;
  constexpr int KS = C::KS;
  using OA = typename C::OA;
  using OB = typename C::OB;
  constexpr int BM = C::BM, BK = C::BK, FM = C::FM, FN = C::FN, LPW = C::LPW;
  constexpr int D = NSG - 1;   // prefetch distance, in the group's own stages
  __shared__ __attribute__((aligned(1024))) char smem_raw[C::SMEM];
  bf16_t *smem = (bf16_t *)smem_raw;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index is the same on every lane: keep it (and every branch on
  // the group) scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wj = wave & 3;
  const int lr = lane & 15, lg = lane >> 4;
  int tm, tn;
  tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, p.raster_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int K = p.K;
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.B, (short)0, (int)p.b_bytes, 0x00020000);

  // The bias starts group 0's accumulators (lane columns wj WTN + 16 j +
  // lane % 16); the two partial tiles are summed once.
  float bcol[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wj * C::WTN + j * 16 + lr;
    bcol[j] = p.bias && grp == 0 && n < p.n_valid ? p.bias[n] : 0.f;
  }
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{bcol[j], bcol[j], bcol[j], bcol[j]};

  bf16_t *ring = smem + grp * C::RING;
  auto At = [&](int slot) { return ring + slot * C::STAGE; };
  auto Bt = [&](int slot) { return ring + slot * C::STAGE + OA::ELEMS; };
  const int nk = (K + BK - 1) / BK;            // global k-stages
  const int nkg = (nk - grp + 1) / 2;           // this group's stages (global 2 i + grp)
  const int iters = (nk + 1) / 2;               // phases pairs, the same for both groups
  // own stage i -> LDS slot i % NSG, global k offset (2 i + grp) BK
  auto issue = [&](int i) {
    const int k0 = (2 * i + grp) * BK;
    OA::template issue<4>(At(i % NSG), rsa, p.lda, m0, k0, p.M, K, wj, lane);
    OB::template issue<4>(Bt(i % NSG), rsb, p.ldb, n0, k0, p.N, K, wj, lane);
  };
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < nkg) issue(i);
  // own stage 0 landed (the loads of stages 1 .. D-1 may still fly)
  wait_vm_stages<LPW>(min(D - 1, nkg - 1));
  pp_barrier();
  if (grp == 1) pp_barrier();   // group 1 runs one phase behind
  bf16x8_t fa[KS][FM], fb[KS][FN];
  for (int i = 0; i < iters; ++i) {
    const bool have = i < nkg;
    // ---- memory phase: this stage's fragments, a later stage's loads
    if (have) {
      const bf16_t *as = At(i % NSG), *bs = Bt(i % NSG);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[s][j] = OB::frag(bs, wj * C::WTN + j * 16, 32 * s, lr, lg);
#pragma unroll
        for (int m = 0; m < FM; ++m) fa[s][m] = OA::frag(as, m * 16, 32 * s, lr, lg);
      }
      if (i + D < nkg) issue(i + D);
      wait_lgkm0();
    }
    pp_barrier();
    // ---- compute phase
    if (have) {
#pragma unroll
      for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int m = 0; m < FM; ++m)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[m][j] = lp_mfma<F16>(fa[s][m], fb[s][j], acc[m][j]);
      // own stage i+1 must have landed before the barrier that opens it;
      // the loads of stages i+2 .. i+D may still fly
      if (i + 1 < nkg) wait_vm_stages<LPW>(min(D - 1, nkg - 2 - i));
    }
    pp_barrier();
  }
  if (grp == 0) pp_barrier();   // both groups have passed the same number

  // ---- the two partial tiles meet in LDS: group 0 stores, group 1 adds
  float *Cs = (float *)smem_raw;
  if (grp == 0) {
#pragma unroll
    for (int m = 0; m < FM; ++m)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Cs[(m * 16 + lg * 4 + r) * C::LDC + wj * C::WTN + j * 16 + lr] = acc[m][j][r];
  }
  __syncthreads();
  if (grp == 1) {
#pragma unroll
    for (int m = 0; m < FM; ++m)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          Cs[(m * 16 + lg * 4 + r) * C::LDC + wj * C::WTN + j * 16 + lr] += acc[m][j][r];
  }
  __syncthreads();
  // ---- epilogue: 4 consecutive columns per thread, rows in turn; column
  // sums (bias gradients) of the stored values go back into the tile and
  // thread t < BN adds up column t.
  constexpr int TPR = BN / 4;
  const int nv = p.n_valid;
  if (p.epi == EPI_RESID && p.vec_out && !p.colsum) {
    // residual products: every residual load of this thread's items is
    // issued first, then the sums are stored -- one memory round trip
    // instead of one per item
    constexpr int ITEMS = (BM * TPR + C::NT - 1) / C::NT;
    float4 rv[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * C::NT;
      const int rr = idx / TPR, cc = (idx % TPR) * 4;
      const int m = m0 + rr, n = n0 + cc;
      rv[it] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (idx < BM * TPR && m < p.M && n + 3 < nv)
        rv[it] = *(const float4 *)(p.resid + (size_t)m * p.ldr + n);
    }
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * C::NT;
      if (idx >= BM * TPR) break;
      const int rr = idx / TPR, cc = (idx % TPR) * 4;
      const int m = m0 + rr, n = n0 + cc;
      if (m >= p.M || n >= nv) continue;
      const float4 v = *(const float4 *)(Cs + rr * C::LDC + cc);
      if (n + 3 < nv) {
        out_store((float *)p.out + (size_t)m * p.ldo + n,
                  make_float4(rv[it].x + v.x, rv[it].y + v.y, rv[it].z + v.z, rv[it].w + v.w));
      } else {
        epilogue4<F16>(p, m, n, v, nv - n);   // the ragged last columns
      }
    }
    return;
  }
  for (int idx = tid; idx < BM * TPR; idx += C::NT) {
    const int rr = idx / TPR, cc = (idx % TPR) * 4;
    const int m = m0 + rr, n = n0 + cc;
    float4 *cp = (float4 *)(Cs + rr * C::LDC + cc);
    if (m >= p.M || n >= nv) {
      if (p.colsum) *cp = make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
    const float4 st = epilogue4<F16>(p, m, n, *cp, nv - n);
    if (p.colsum) *cp = st;
  }
  if (p.colsum) {
    lds_barrier();
    if (tid < BN && n0 + tid < nv)
      unsafeAtomicAdd(&p.colsum[n0 + tid], column_sum<BM, C::LDC>(Cs, tid));
  }
}

template <int BN, int NSG, int BKP>
int launch_pp(tt_ctx *ctx, const GemmArgs &g) {
  using C = PPCfg<BN, NSG, BKP>;
  GemmParams p{};
  p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.epi = g.epi; p.out = g.out; p.ldo = g.ldo; p.out_bf16 = g.out_bf16 ? 1 : 0;
  p.bias = g.bias; p.resid = g.resid; p.ldr = g.ldr; p.aux = g.aux; p.ldx = g.ldx;
  p.n_valid = g.n_valid > 0 ? min(g.n_valid, g.N) : g.N;
  p.vec_out = gemm_vec_out(g) ? 1 : 0;
  p.colsum = g.colsum;
  p.raster_n = g.raster == 2 ? 1 : 0;
  p.a_bytes = (uint32_t)gemm_extent_bytes(true, g.M, g.K, g.lda);
  p.b_bytes = (uint32_t)gemm_extent_bytes(true, g.N, g.K, g.ldb);
  p.tiles_m = (g.M + C::BM - 1) / C::BM;
  p.tiles_n = (g.N + BN - 1) / BN;
  p.k_chunk = g.K;
  const int tiles = p.tiles_m * p.tiles_n;
  static char names[2][80];
  char *name = names[g.f16 ? 1 : 0];
  if (!name[0])
    snprintf(name, sizeof names[0], "gemm_pp_kernel<%d, %d, %d, %s>", BN, NSG, BKP,
             g.f16 ? "true" : "false");
  tt_prof_scope prof(ctx, name, 2.0 * g.M * g.N * g.K, gemm_bytes(g));
  if (g.f16)
    hipLaunchKernelGGL((gemm_pp_kernel<BN, NSG, BKP, true>), dim3(tiles), dim3(C::NT), 0, ctx->stream, p);
  else
    hipLaunchKernelGGL((gemm_pp_kernel<BN, NSG, BKP, false>), dim3(tiles), dim3(C::NT), 0, ctx->stream, p);
  return tt_check_launch(ctx, "gemm_pp");
}

// out (+)= sum of the split partials (accumulate = 0: out is overwritten).
__global__ void __launch_bounds__(256) splitk_reduce_kernel(float *__restrict__ out, int ldo,
                                                             const float *__restrict__ ws, int M,
                                                             int N, int split, int accumulate) {
  const size_t mn = (size_t)M * N;
  const size_t n4 = mn / 4;
  const size_t stride = (size_t)gridDim.x * 256;
  if (N % 4 == 0 && ldo % 4 == 0) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
      float4 s = ((const float4 *)ws)[i];
      for (int z = 1; z < split; ++z) {
        float4 t = ((const float4 *)(ws + z * mn))[i];
        s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
      }
      const size_t e = i * 4;
      const int m = (int)(e / N), n = (int)(e % N);
      float4 *o = (float4 *)(out + (size_t)m * ldo + n);
      if (accumulate) {
        const float4 c = *o;
        s.x += c.x; s.y += c.y; s.z += c.z; s.w += c.w;
      }
      *o = s;
    }
  } else {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < mn; i += stride) {
      float s = ws[i];
      for (int z = 1; z < split; ++z) s += ws[z * mn + i];
      float *o = out + (i / N) * ldo + i % N;
      *o = accumulate ? *o + s : s;
    }
  }
}

// --------------------------------------------------------------------------
// Skinny products (at most 16 rows, both operands k-major): the single-token
// decode step, where every weight is read once per step and the product is
// bound by that read.  One workgroup per 16 output columns; its 4 waves take
// interleaved 32-wide slices of K, each accumulating the 16 x 16 tile with
// v_mfma_f32_16x16x32_bf16 straight from global memory (rows past M and k
// past K read zero through the buffer range checks); the 4 partial tiles
// are added in LDS and the usual epilogue runs on 4-column groups.
// --------------------------------------------------------------------------
constexpr int SK_BATCH = 8;   // MFMA steps whose loads are issued together

__global__ void __launch_bounds__(256) gemm_skinny_kernel(GemmParams p) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)p.a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc((void *)p.B, (short)0, (int)p.b_bytes, 0x00020000);
  const int m = lr, n = n0 + lr;
  const bool mok = m < p.M, nok = n < p.N;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int nsteps = (p.K + 31) / 32;
  for (int s0 = wave; s0 < nsteps; s0 += 4 * SK_BATCH) {
    uint4 fa[SK_BATCH], fb[SK_BATCH];
#pragma unroll
    for (int j = 0; j < SK_BATCH; ++j) {
      const int k = (s0 + 4 * j) * 32 + 8 * lg;
      const bool kok = s0 + 4 * j < nsteps && k < p.K;
      const uint32_t oa = (mok && kok) ? (uint32_t)(((size_t)m * p.lda + k) * 2) : OOB;
      const uint32_t ob = (nok && kok) ? (uint32_t)(((size_t)n * p.ldb + k) * 2) : OOB;
      fa[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsa, oa, 0, 0));
      fb[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsb, ob, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < SK_BATCH; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[j]),
                                                     __builtin_bit_cast(bf16x8_t, fb[j]), acc,
                                                     0, 0, 0);
  }
  __shared__ float part[4][16][17];
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][lg * 4 + r][lr] = acc[r];
  __syncthreads();
  if (tid >= 64) return;
  const int row = tid >> 2, cg = (tid & 3) * 4;
  const int nn = n0 + cg, nv = p.n_valid;
  if (row >= p.M || nn >= nv) return;
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = (part[0][row][cg + q] + part[1][row][cg + q]) + (part[2][row][cg + q] + part[3][row][cg + q]);
    if (p.bias && nn + q < nv) v[q] += p.bias[nn + q];
  }
  epilogue4(p, row, nn, make_float4(v[0], v[1], v[2], v[3]), nv - nn);
}

int launch_skinny(tt_ctx *ctx, const GemmArgs &g) {
  GemmParams p{};
  p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.epi = g.epi; p.out = g.out; p.ldo = g.ldo; p.out_bf16 = g.out_bf16 ? 1 : 0;
  p.bias = g.bias; p.resid = g.resid; p.ldr = g.ldr; p.aux = g.aux; p.ldx = g.ldx;
  p.n_valid = g.n_valid > 0 ? min(g.n_valid, g.N) : g.N;
  p.vec_out = gemm_vec_out(g) ? 1 : 0;
  p.a_bytes = (uint32_t)gemm_extent_bytes(true, g.M, g.K, g.lda);
  p.b_bytes = (uint32_t)gemm_extent_bytes(true, g.N, g.K, g.ldb);
  tt_prof_scope prof(ctx, "gemm_skinny_kernel", 2.0 * g.M * g.N * g.K, gemm_bytes(g));
  hipLaunchKernelGGL(gemm_skinny_kernel, dim3((g.N + 15) / 16), dim3(256), 0, ctx->stream, p);
  return tt_check_launch(ctx, "gemm_skinny");
}

}  // namespace

// Host guard: the buffer-load path needs every operand extent below the OOB
// offset, and K % 8 == 0 whenever an operand is k-major.  A k-major row is
// read in 8-element chunks; with K % 8 != 0 the last chunk of a row would
// reach k >= K, i.e. the next row or bytes past the tensor, and a zero in
// the partner operand does not cancel an inf / NaN there (0 * inf = NaN).
// Such products take the generic kernels.
bool tt_gemm_bf16_ok(const GemmArgs &g) {
  if (gemm_extent_bytes(g.a_kmajor, g.M, g.K, g.lda) >= OOB) return false;
  if (gemm_extent_bytes(g.b_kmajor, g.N, g.K, g.ldb) >= OOB) return false;
  return g.K % 8 == 0 || (!g.a_kmajor && !g.b_kmajor);
}

// Tiles (8 waves, direct-to-LDS v3 kernel unless noted), chosen from sweeps
// of the GPT-2 step's shapes on MI355X:
//  * k-major x k-major products (dX = dY W, forward GEMMs against transposed
//    weights, the LM head):
//      N < 1536 (the N = 768 products), M > 128: the ping-pong kernel,
//        128 x 192, two 64-deep stages per group (gemm_pp_kernel)
//    and otherwise:
//      K <= 1024, exactly 256 tiles of 256 x 288 (the qkv forward at 8192
//      tokens)                                  256 x 288, BK 32, 3 stages
//                                               (one workgroup per CU)
//      K >= 8192 (LM-head dH)                   128 x 192, BK 64, 3 stages
//      >= 512 tiles of 256 x 128:  GELU-backward epilogue -> 128 x 192, BK 64,
//                                  2 stages; others -> 256 x 128, BK 32, 3
//                                  stages (two workgroups per CU)
//      fewer tiles (N = 768): K >= 2304 -> 128 x 192, BK 64, 3 stages (256
//                             tiles fill the 256 CUs where 256 x 128 gives
//                             192); else 256 x 128, BK 64, 3 stages
//    (ranked with operands arriving cold from HBM, as in the step; with
//    cache-resident operands the ranking differs)
//  * one row-major operand: the register-prefetch v2 kernel, 256 x 128;
//  * weight gradients: 256 x 128, BK 32, 3 stages (below; two workgroups
//    per CU).
// Tile order within an XCD: m fastest (neighbouring workgroups share B
// panels) except on the 256 x 128 BK-32 path, where n fastest (shared A
// panels) measured faster inside the step.
// Weight gradients (EPI_ACCUM, output += product) never use atomics: one
// split accumulates with a plain read-modify-write (a workgroup owns its
// output tile); several splits write fp32 partials to arena scratch, then
// one coalesced pass adds them into the output.  The split is the largest
// that keeps the grid within 512 workgroups (two per CU), at most 16, with at
// least 256 of K per split.
int tt_gemm_bf16(tt_ctx *ctx, const GemmArgs &g) {
  const long tiles = (long)((g.M + 255) / 256) * ((g.N + 127) / 128);
  if (g.M <= 16 && !g.f16 && g.a_kmajor && g.b_kmajor && !g.colsum && g.K % 8 == 0 &&
      (g.epi == EPI_STORE || g.epi == EPI_GELU || g.epi == EPI_RESID))
    return launch_skinny(ctx, g);
  if (g.epi != EPI_ACCUM) {
    if (g.colsum && !(g.a_kmajor && g.b_kmajor))
      return tt_set_error(ctx, TT_EINVAL, "gemm_bf16: column sums need the k-major kernel");
    if (!(g.a_kmajor && g.b_kmajor)) return launch<256, 128, 4, 2>(ctx, g, 1);
    // the narrow products (N = 768: projections, down-projection, every dX
    // but the GELU-backward one, the LM-head dH): ping-pong tile
    if (g.N < 1536 && g.M > 128) return launch_pp<192, 2, 64>(ctx, g);
    // Products whose 256 x 128 grid leaves a short second round (the qkv
    // forward: 576 tiles on 512 slots, the last 64 running alone) take
    // 256 x 288 tiles when those fill the GPU in exactly one round (one
    // workgroup per CU): 48 against 54 us at M = 8192, N = 2304, K = 768.
    if (g.K <= 1024 && g.M % 256 == 0 && g.N % 288 == 0 && (long)(g.M / 256) * (g.N / 288) == 256)
      return launch3<256, 288, 32, 4, 2, 3>(ctx, g, 1);
    if (g.K >= 8192) return launch3<128, 192, 64, 2, 4, 3>(ctx, g, 1);
    if (tiles >= 512) {
      if (g.epi == EPI_GELU_BWD) return launch3<128, 192, 64, 2, 4, 2>(ctx, g, 1);
      GemmArgs h = g;
      if (h.raster == 0) h.raster = 2;
      return launch3<256, 128, 32, 4, 2, 3>(ctx, h, 1);
    }
    if (g.K >= 2304) return launch3<128, 192, 64, 2, 4, 3>(ctx, g, 1);
    return launch3<256, 128, 64, 4, 2, 3>(ctx, g, 1);
  }
  const int kb = (g.K + 31) / 32;
  auto rounded = [&](int split) {  // the split launch3 will run (whole k-blocks)
    const int per = (kb + split - 1) / split;
    return (kb + per - 1) / per;
  };
  int split = rounded((int)std::max<long>(1, std::min<long>(512 / tiles, std::min(kb / 8, 16))));
  if (g.split_k > 0) split = rounded(g.split_k);
  GemmArgs h = g;
  if (h.raster == 0) h.raster = 1;
  if (split == 1) {
    h.epi = g.overwrite ? EPI_STORE : EPI_STORE_ACC;
    h.out_bf16 = false;
    h.bias = nullptr;
    return launch3<256, 128, 32, 4, 2, 3>(ctx, h, 1);
  }
  tt_scratch_scope scope(ctx);
  void *ws;
  TT_TRY(tt_arena_alloc(ctx, (size_t)split * g.M * g.N * 4, &ws));
  h.epi = EPI_STORE;
  h.out = ws;
  h.ldo = g.N;
  h.out_bf16 = false;
  h.bias = nullptr;
  // split is already what launch3 runs (whole k-blocks per split), so the
  // reduction sums exactly the partials written.
  TT_TRY((launch3<256, 128, 32, 4, 2, 3>(ctx, h, split, (size_t)g.M * g.N)));
  const size_t work = (size_t)g.M * g.N / 4;
  const int blocks = (int)std::min<size_t>((work + 255) / 256, 4096);
  tt_prof_scope prof(ctx, "splitk_reduce_kernel", 0.0,
                     (split + (g.overwrite ? 1.0 : 2.0)) * g.M * g.N * 4.0);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(blocks), dim3(256), 0, ctx->stream, (float *)g.out,
                     g.ldo, (const float *)ws, g.M, g.N, split, g.overwrite ? 0 : 1);
  return tt_check_launch(ctx, "splitk_reduce");
}

// ------------------------------------------------------------ grouped launch
// The products of a group share one kernel configuration (the weight-gradient
// tile: 256 x 128, BK 32, 3 stages, both operands read with the LDS transpose)
// and one reduction length; each workgroup owns one output tile of one
// product.  Run as one launch, the 48 weight gradients of a 12-layer model
// and the token-table gradient fill the machine without splitting K.
// Tile of the grouped launch (BM, BN, BK, waves along M, along N, stages);
// measured inside the GPT-2 124M step against 256x128 BK 32/64 with 2-3
// stages, 256x256 and 128x256 (3 stages gain once the transpose reads no
// longer drain the ring).
#ifndef TT_GROUP_TILE
#define TT_GROUP_TILE 256, 128, 32, 4, 2, 3
#endif
namespace {
template <int BM, int BN, int BKV, int WM, int WN, int NS>
struct GroupTile {
  static constexpr int bm = BM, bn = BN, bk = BKV, wm = WM, wn = WN, ns = NS;
};
using GT = GroupTile<TT_GROUP_TILE>;
constexpr int GBM = GT::bm, GBN = GT::bn, GBK = GT::bk;
}

namespace {
// Validate the entries for reduction lengths up to k_max and fill in their
// tile fields; tiles, mn2, bytes_k, bytes_out receive the totals.
int group_fill(tt_ctx *ctx, std::vector<GemmGroupEntry> &t, int k_max, int &tiles, double &mn2,
               double &bytes_k, double &bytes_out) {
  tiles = 0;
  mn2 = bytes_k = bytes_out = 0;
  for (auto &e : t) {
    TT_REQUIRE(ctx, e.A && e.B && e.out && e.M > 0 && e.N > 0, "gemm_group: bad entry");
    TT_REQUIRE(ctx, e.lda >= e.M && e.ldb >= e.N && e.ldo >= e.N, "gemm_group: bad leading dims");
    TT_REQUIRE(ctx, tt_aligned16(e.A) && tt_aligned16(e.B) && e.lda % 8 == 0 && e.ldb % 8 == 0,
               "gemm_group: operand rows must be 16-byte aligned");
    TT_REQUIRE(ctx, gemm_extent_bytes(false, e.M, k_max, e.lda) < OOB &&
                        gemm_extent_bytes(false, e.N, k_max, e.ldb) < OOB,
               "gemm_group: operand too large for buffer addressing");
    e.tiles_m = (e.M + GBM - 1) / GBM;
    e.tiles_n = (e.N + GBN - 1) / GBN;
    e.tile0 = tiles;
    e.vec_out = ((uintptr_t)e.out % 16 == 0 && e.ldo % 4 == 0) ? 1 : 0;
    // Tile order: neighbouring workgroups share the panel of the larger
    // operand (n fastest when A has far more columns than B, as for the token
    // table: its [tokens, vocabulary] gradient panel is then read once).
    e.raster_n = e.M >= 4 * e.N ? 1 : 0;
    tiles += e.tiles_m * e.tiles_n;
    mn2 += 2.0 * e.M * e.N;
    bytes_k += 2.0 * (e.M + e.N);
    bytes_out += 4.0 * e.M * e.N;
  }
  return TT_OK;
}
}  // namespace

int tt_gemm_group_plan(tt_ctx *ctx, const GemmGroupEntry *entries, int n, int k_max,
                       GemmGroup *out, bool f16) {
  TT_REQUIRE(ctx, entries && out && n > 0 && k_max > 0, "gemm_group: bad arguments");
  std::vector<GemmGroupEntry> t(entries, entries + n);
  int tiles = 0;
  double mn2 = 0, bytes_k = 0, bytes_out = 0;
  TT_TRY(group_fill(ctx, t, k_max, tiles, mn2, bytes_k, bytes_out));
  const int grid = (tiles + 7) / 8 * 8;
  TT_REQUIRE(ctx, grid < 0xffff && n < 0xffff, "gemm_group: too many tiles");
  std::vector<uint16_t> map(grid, 0xffff);
  for (int i = 0; i < n; ++i)
    for (int k = 0; k < t[i].tiles_m * t[i].tiles_n; ++k) map[t[i].tile0 + k] = (uint16_t)i;
  void *pt, *pm;
  TT_TRY(tt_arena_alloc(ctx, t.size() * sizeof(GemmGroupEntry), &pt));
  TT_TRY(tt_arena_alloc(ctx, map.size() * sizeof(uint16_t), &pm));
  hipError_t e1 = hipMemcpyAsync(pt, t.data(), t.size() * sizeof(GemmGroupEntry),
                                 hipMemcpyHostToDevice, ctx->stream);
  hipError_t e2 = hipMemcpyAsync(pm, map.data(), map.size() * sizeof(uint16_t),
                                 hipMemcpyHostToDevice, ctx->stream);
  if (e1 != hipSuccess || e2 != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "gemm_group: table upload failed");
  // the host vectors die here: make sure the copies have read them
  hipError_t e3 = hipStreamSynchronize(ctx->stream);
  if (e3 != hipSuccess) return tt_set_error(ctx, TT_EHIP, "gemm_group: %s", hipGetErrorString(e3));
  out->table = (GemmGroupEntry *)pt;
  out->map = (uint16_t *)pm;
  out->n = n;
  out->tiles = tiles;
  out->grid = grid;
  out->mn2 = mn2;
  out->bytes_k = bytes_k;
  out->bytes_out = bytes_out;
  out->f16 = f16;
  return TT_OK;
}

int tt_gemm_group_update(tt_ctx *ctx, GemmGroup &g, const GemmGroupEntry *entries, int n,
                         int k_max) {
  TT_REQUIRE(ctx, g.table && g.map && entries && n == g.n && k_max > 0,
             "gemm_group_update: not planned for %d products", n);
  std::vector<GemmGroupEntry> t(entries, entries + n);
  int tiles = 0;
  double mn2 = 0, bytes_k = 0, bytes_out = 0;
  TT_TRY(group_fill(ctx, t, k_max, tiles, mn2, bytes_k, bytes_out));
  TT_REQUIRE(ctx, tiles == g.tiles && mn2 == g.mn2, "gemm_group_update: product shapes changed");
  hipError_t e = hipMemcpyAsync(g.table, t.data(), t.size() * sizeof(GemmGroupEntry),
                                hipMemcpyHostToDevice, ctx->stream);
  // the host vector dies here: make sure the copy has read it
  if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "gemm_group_update: %s", hipGetErrorString(e));
  g.bytes_k = bytes_k;
  g.bytes_out = bytes_out;
  return TT_OK;
}

int tt_gemm_group_run(tt_ctx *ctx, const GemmGroup &g, int K, bool accumulate) {
  TT_REQUIRE(ctx, g.table && g.map && g.grid > 0 && K > 0, "gemm_group: not planned");
  GemmParams p{};
  p.K = K;
  p.k_chunk = (K + GBK - 1) / GBK * GBK;
  p.epi = accumulate ? EPI_STORE_ACC : EPI_STORE;
  p.out_bf16 = 0;
  p.raster_n = 0;
  p.group = g.table;
  p.group_map = g.map;
  static char names[2][112];
  char *name = names[g.f16 ? 1 : 0];
  if (!name[0])
    snprintf(name, sizeof names[0], "gemm_bf16_v3_kernel<%d, %d, %d, %d, %d, %d, false, false, true, %s>",
             GT::bm, GT::bn, GT::bk, GT::wm, GT::wn, GT::ns, g.f16 ? "true" : "false");
  tt_prof_scope prof(ctx, name, g.mn2 * K, g.bytes_k * K + g.bytes_out);
  if (g.f16)
    hipLaunchKernelGGL(
        (gemm_bf16_v3_kernel<GBM, GBN, GBK, GT::wm, GT::wn, GT::ns, false, false, true, true>),
        dim3(g.grid), dim3(64 * GT::wm * GT::wn), 0, ctx->stream, p);
  else
    hipLaunchKernelGGL(
        (gemm_bf16_v3_kernel<GBM, GBN, GBK, GT::wm, GT::wn, GT::ns, false, false, true, false>),
        dim3(g.grid), dim3(64 * GT::wm * GT::wn), 0, ctx->stream, p);
  return tt_check_launch(ctx, "gemm_group");
}
