// MFMA GEMM for gfx950 with fused epilogues.
//
// Computes C[m,n] = sum_k A(m,k) B(k,n) — the tinytorch page's MatMul
// (section 3 item 3) and its two backward products dA = dC·Bᵀ, dB = Aᵀ·dC —
// on the matrix cores: v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulation) or v_mfma_f32_16x16x4_f32 (fp32 mode).  The Forge page
// ("核心组件清单" and the GEMM discussion) blocks GEMM over the cache levels;
// here the levels are HBM -> LDS (double-buffered tiles) -> registers (MFMA
// fragments).
//
// Operand majority.  Either operand can be "k-major" (the reduction index is
// contiguous) or not.  Tiles are always stored k-contiguous in LDS, because an
// MFMA lane reads KPL consecutive k values of one row (A) or one column (B).
// A non-k-major source is transposed on its way into LDS: each thread loads
// two k rows of 8 contiguous values (bf16) and writes 8 packed dwords.
//
// MFMA fragment layout used (16x16 blocks, wave64): lane l holds row l%16 of
// A and column l%16 of B for the k slots of lane group l/16; the accumulator
// holds D[4*(l/16)+r][l%16], r = 0..3.
#include "gemm_common.h"

namespace {

using namespace tt_gemm_detail;

template <typename T> struct MfmaTraits;
template <> struct MfmaTraits<bf16_t> {
  static constexpr int KPL = 8;    // k values per lane per MFMA
  static constexpr int KSTEP = 32; // k per MFMA
  static constexpr int VEC = 8;    // elements per 16-byte global load
  typedef bf16x8_t frag_t;
  __device__ __forceinline__ static f32x4_t mfma(frag_t a, frag_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MfmaTraits<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 4;
  static constexpr int VEC = 4;
  typedef float frag_t;
  __device__ __forceinline__ static f32x4_t mfma(frag_t a, frag_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Tile shape: BM x BN block, BK deep, WM x WN waves.
template <typename T, int BM, int BN, int BK, int WM, int WN>
struct Tile {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int PAD = 16 / sizeof(T);      // keeps rows 16-byte aligned, spreads banks
  static constexpr int LDK = BK + PAD;            // LDS row length (elements)
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / 16, FN = WTN / 16;
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
};

// ------------------------------------------------------------------ loaders
// Load one BM(or BN) x BK operand tile into registers, then store to LDS.
// ROWS: tile rows (m or n extent), the k extent is BK.
template <typename T, int ROWS, int BK, int NT, bool KMAJOR, bool VECLD>
struct TileLoader {
  static constexpr int VEC = MfmaTraits<T>::VEC;
  // k-major vector loads: ROWS*BK/VEC vectors.  non-k-major bf16 loads are
  // pairs of k rows (2 vectors); fp32 single vectors.
  static constexpr int KROWS = (sizeof(T) == 2) ? 2 : 1;
  static constexpr int UNITS = KMAJOR ? (ROWS * BK / VEC) : (ROWS * BK / (VEC * KROWS));
  static constexpr int PER_THREAD = (UNITS + NT - 1) / NT;
  static constexpr int LOADS = KMAJOR ? PER_THREAD : PER_THREAD * KROWS;
  uint4 reg[VECLD ? LOADS : 1];
  T sreg[VECLD ? 1 : (ROWS * BK + NT - 1) / NT];

  // Element (r, k) of the operand (r = row of A / column of B).
  __device__ __forceinline__ static T get(const T *p, int ld, int r, int k, int R, int K) {
    if (r >= R || k >= K) return T(0);
    return KMAJOR ? p[(size_t)r * ld + k] : p[(size_t)k * ld + r];
  }

  // Pack VEC elements (element i read by f(i), zero when !ok(i)) into a uint4
  // without an addressable temporary (keeps everything in registers).
  template <typename F>
  __device__ __forceinline__ static uint4 gather_vec(F f) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (sizeof(T) == 2) {
        uint32_t lo = f(2 * q), hi = f(2 * q + 1);
        w[q] = lo | (hi << 16);
      } else {
        w[q] = f(q);
      }
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ __forceinline__ static uint32_t bits(T v) {
    if constexpr (sizeof(T) == 2) return (uint32_t)v;
    else return __float_as_uint(v);
  }

  __device__ __forceinline__ static uint4 load_vec_kmajor(const T *p, int ld, int r, int k, int R,
                                                          int K) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < R) {
      const T *row = p + (size_t)r * ld;
      if (k + VEC <= K) {
        v = *(const uint4 *)(row + k);
      } else if (k < K) {
        v = gather_vec([&](int i) { return (k + i < K) ? bits(row[k + i]) : 0u; });
      }
    }
    return v;
  }
  __device__ __forceinline__ static uint4 load_vec_rmajor(const T *p, int ld, int k, int r, int R,
                                                          int K) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < K) {
      const T *row = p + (size_t)k * ld;
      if (r + VEC <= R) {
        v = *(const uint4 *)(row + r);
      } else if (r < R) {
        v = gather_vec([&](int i) { return (r + i < R) ? bits(row[r + i]) : 0u; });
      }
    }
    return v;
  }

  // Unit u of a non-k-major tile: 4 consecutive units cover 4 x VEC
  // consecutive rows (a 64-byte global segment), then k advances.
  __device__ __forceinline__ static void unit_rmajor(int u, int &kp, int &rc) {
    constexpr int RC = ROWS / VEC;   // row chunks
    constexpr int KP = BK / KROWS;   // k groups
    int lo = u % 4, rest = u / 4;
    kp = rest % KP;
    rc = (rest / KP) * 4 + lo;
    (void)RC;
  }

  __device__ __forceinline__ void load(const T *p, int ld, int r0, int k0, int R, int K, int tid) {
    if constexpr (VECLD) {
      if constexpr (KMAJOR) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
          int u = tid + i * NT;
          if (UNITS % NT == 0 || u < UNITS) {
            int r = u / (BK / VEC), kc = u % (BK / VEC);
            reg[i] = load_vec_kmajor(p, ld, r0 + r, k0 + kc * VEC, R, K);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
          int u = tid + i * NT;
          if (UNITS % NT == 0 || u < UNITS) {
            int kp, rc;
            unit_rmajor(u, kp, rc);
#pragma unroll
            for (int j = 0; j < KROWS; ++j)
              reg[i * KROWS + j] =
                  load_vec_rmajor(p, ld, k0 + kp * KROWS + j, r0 + rc * VEC, R, K);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < (ROWS * BK + NT - 1) / NT; ++i) {
        int e = tid + i * NT;
        if (e < ROWS * BK) {
          int r = e / BK, k = e % BK;
          sreg[i] = get(p, ld, r0 + r, k0 + k, R, K);
        }
      }
    }
  }

  template <int LDK>
  __device__ __forceinline__ void store(T *s, int tid) const {
    if constexpr (VECLD) {
      if constexpr (KMAJOR) {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
          int u = tid + i * NT;
          if (UNITS % NT == 0 || u < UNITS) {
            int r = u / (BK / VEC), kc = u % (BK / VEC);
            *(uint4 *)(s + r * LDK + kc * VEC) = reg[i];
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < PER_THREAD; ++i) {
          int u = tid + i * NT;
          if (UNITS % NT == 0 || u < UNITS) {
            int kp, rc;
            unit_rmajor(u, kp, rc);
            if constexpr (sizeof(T) == 2) {
              const uint32_t *a = (const uint32_t *)&reg[i * 2];
              const uint32_t *b = (const uint32_t *)&reg[i * 2 + 1];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                // rows rc*8 + 2q and rc*8 + 2q + 1; k = 2kp, 2kp+1
                uint32_t lo = (a[q] & 0xffffu) | (b[q] << 16);
                uint32_t hi = (a[q] >> 16) | (b[q] & 0xffff0000u);
                *(uint32_t *)(s + (rc * 8 + 2 * q) * LDK + 2 * kp) = lo;
                *(uint32_t *)(s + (rc * 8 + 2 * q + 1) * LDK + 2 * kp) = hi;
              }
            } else {
              const float *a = (const float *)&reg[i];
#pragma unroll
              for (int q = 0; q < 4; ++q) s[(rc * 4 + q) * LDK + kp] = a[q];
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < (ROWS * BK + NT - 1) / NT; ++i) {
        int e = tid + i * NT;
        if (e < ROWS * BK) {
          int r = e / BK, k = e % BK;
          s[r * LDK + k] = sreg[i];
        }
      }
    }
  }
};

template <typename T, int BM, int BN, int BK, int WM, int WN, bool A_KM, bool B_KM, bool VECLD>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_kernel(GemmParams p) {
  using TL = Tile<T, BM, BN, BK, WM, WN>;
  using MT = MfmaTraits<T>;
  constexpr int NT = TL::NT, LDK = TL::LDK, FM = TL::FM, FN = TL::FN;
  __shared__ __attribute__((aligned(16))) T smem[2 * (TL::A_ELEMS + TL::B_ELEMS)];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Tile order: consecutive workgroups walk n first so they share A rows.
  const int tile = blockIdx.x;
  const int tm = tile / p.tiles_n, tn = tile % p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = blockIdx.z * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);

  const T *A = (const T *)p.A;
  const T *B = (const T *)p.B;
  TileLoader<T, BM, BK, NT, A_KM, VECLD> la;
  TileLoader<T, BN, BK, NT, B_KM, VECLD> lb;

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  T *As0 = smem, *Bs0 = smem + TL::A_ELEMS;
  T *As1 = smem + TL::A_ELEMS + TL::B_ELEMS, *Bs1 = As1 + TL::A_ELEMS;

  const int nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) {
    la.load(A, p.lda, m0, kbeg, p.M, kend, tid);
    lb.load(B, p.ldb, n0, kbeg, p.N, kend, tid);
    la.template store<LDK>(As0, tid);
    lb.template store<LDK>(Bs0, tid);
  }
  __syncthreads();

  const int lr = lane & 15, lg = lane >> 4;
  for (int it = 0; it < nk; ++it) {
    T *As = (it & 1) ? As1 : As0;
    T *Bs = (it & 1) ? Bs1 : Bs0;
    const bool more = it + 1 < nk;
    if (more) {
      int k0 = kbeg + (it + 1) * BK;
      la.load(A, p.lda, m0, k0, p.M, kend, tid);
      lb.load(B, p.ldb, n0, k0, p.N, kend, tid);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += MT::KSTEP) {
      typename MT::frag_t fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *(const typename MT::frag_t *)(As + (wm * TL::WTM + i * 16 + lr) * LDK + kk +
                                               lg * MT::KPL);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *(const typename MT::frag_t *)(Bs + (wn * TL::WTN + j * 16 + lr) * LDK + kk +
                                               lg * MT::KPL);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = MT::mfma(fa[i], fb[j], acc[i][j]);
    }
    if (more) {
      T *An = (it & 1) ? As0 : As1;
      T *Bn = (it & 1) ? Bs0 : Bs1;
      la.template store<LDK>(An, tid);
      lb.template store<LDK>(Bn, tid);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // Stage the fp32 C tile through LDS (the operand buffers are free now), then
  // apply the epilogue cooperatively: each thread owns 4 consecutive columns,
  // so bias / residual / aux reads and the output writes are row-coalesced.
  constexpr int LDC = BN + 4;
  static_assert(BM * LDC * 4 <= (int)sizeof(smem), "C tile does not fit in LDS");
  float *Cs = (float *)smem;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        Cs[(wm * TL::WTM + i * 16 + lg * 4 + r) * LDC + wn * TL::WTN + j * 16 + lr] = acc[i][j][r];
  __syncthreads();
  constexpr int TPR = BN / 4;            // threads per row
  constexpr int RPP = NT / TPR;          // rows per pass
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
  for (int rr = tid / TPR; rr < BM; rr += RPP) {
    const int m = m0 + rr;
    if (m >= p.M || n >= nv) continue;
    float4 v = *(const float4 *)(Cs + rr * LDC + cc);
    v.x += bias.x; v.y += bias.y; v.z += bias.z; v.w += bias.w;
    epilogue4(p, m, n, v, nv - n);
  }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool A_KM, bool B_KM, bool VECLD>
int launch_gemm(tt_ctx *ctx, const GemmArgs &g, int split) {
  GemmParams p{};
  p.A = g.A; p.lda = g.lda; p.B = g.B; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.epi = g.epi; p.out = g.out; p.ldo = g.ldo; p.out_bf16 = g.out_bf16 ? 1 : 0;
  p.bias = g.bias; p.resid = g.resid; p.ldr = g.ldr; p.aux = g.aux; p.ldx = g.ldx;
  p.n_valid = g.n_valid > 0 ? min(g.n_valid, g.N) : g.N;
  p.vec_out = gemm_vec_out(g) ? 1 : 0;
  p.tiles_m = (g.M + BM - 1) / BM;
  p.tiles_n = (g.N + BN - 1) / BN;
  int kb = (g.K + BK - 1) / BK;
  int per = (kb + split - 1) / split;
  p.k_chunk = per * BK;
  split = (kb + per - 1) / per;
  dim3 grid(p.tiles_m * p.tiles_n, 1, split);
  tt_prof_scope prof(ctx, sizeof(T) == 2 ? "gemm_kernel<bf16>" : "gemm_kernel<f32>",
                     2.0 * g.M * g.N * g.K, 0.0);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, A_KM, B_KM, VECLD>), grid,
                     dim3(64 * WM * WN), 0, ctx->stream, p);
  return tt_check_launch(ctx, "gemm");
}

template <typename T, int BM, int BN, int BK, int WM, int WN>
int dispatch_layout(tt_ctx *ctx, const GemmArgs &g, int split, bool vec) {
#define TT_G(AK, BKM, V) \
  if (g.a_kmajor == AK && g.b_kmajor == BKM && vec == V) \
    return launch_gemm<T, BM, BN, BK, WM, WN, AK, BKM, V>(ctx, g, split);
  TT_G(true, true, true) TT_G(true, false, true) TT_G(false, true, true) TT_G(false, false, true)
  TT_G(true, true, false) TT_G(true, false, false) TT_G(false, true, false)
  TT_G(false, false, false)
#undef TT_G
  return TT_EINVAL;
}

}  // namespace

int tt_gemm(tt_ctx *ctx, tt_mode mode, const GemmArgs &g) {
  TT_REQUIRE(ctx, g.M > 0 && g.N > 0 && g.K > 0, "gemm: empty shape %d %d %d", g.M, g.N, g.K);
  TT_REQUIRE(ctx, g.A && g.B && g.out, "gemm: NULL operand");
  const int esz = tt_lowp(mode) ? 2 : 4;
  const int vecn = 16 / esz;
  bool vec = tt_aligned16(g.A) && tt_aligned16(g.B) && (g.lda % vecn == 0) &&
             (g.ldb % vecn == 0);
  // fp32 products whose 128 x 128 tile grid would leave CUs idle (the
  // single-block workload has 1024 tokens: 48 to 144 such tiles for 256 CUs)
  // take 64 x 64 tiles: four times the workgroups, each of four waves of
  // 32 x 32.
  const bool small_f32 = mode == TT_F32 && ((g.M + 127) / 128) * ((g.N + 127) / 128) < 256;
  const int tb = small_f32 ? 64 : 128;
  int split = 1;
  if (g.epi == EPI_ACCUM) {
    // Split the reduction when the output tile grid is too small to fill 256
    // CUs; partial sums meet in the float32 output through atomics.
    int tiles = ((g.M + tb - 1) / tb) * ((g.N + tb - 1) / tb);
    int kb = (g.K + 63) / 64;
    split = 1;
    while (tiles * split < 512 && split * 2 <= kb / 4) split *= 2;
    if (g.split_k > 0) split = g.split_k;
  }
  // Column sums of the output (g.colsum) are fused into the epilogue of the
  // direct-to-LDS bf16 kernel; every other path sums the stored output after.
  const bool fast = tt_lowp(mode) && vec && tt_gemm_bf16_ok(g);
  if (mode == TT_FP16 && !fast)
    return tt_set_error(ctx, TT_EUNSUPPORTED,
                        "gemm(fp16): operands need 16-byte aligned rows (lda, ldb multiples of 8)");
  if (g.epi == EPI_ACCUM && g.overwrite && !fast) {
    // the generic kernels accumulate with atomics: clear the output first
    TT_REQUIRE(ctx, g.ldo == g.N, "gemm: overwrite needs a dense output");
    TT_TRY(tt_fill_f32(ctx, (float *)g.out, (size_t)g.M * g.N, 0.f));
  }
  const bool fused_sum = fast && g.epi != EPI_ACCUM && g.a_kmajor && g.b_kmajor;
  GemmArgs h = g;
  h.f16 = mode == TT_FP16;
  if (!fused_sum) h.colsum = nullptr;
  if (fast)
    TT_TRY(tt_gemm_bf16(ctx, h));
  else if (mode == TT_BF16)
    TT_TRY((dispatch_layout<bf16_t, 128, 128, 64, 2, 2>(ctx, h, split, vec)));
  else if (small_f32)
    TT_TRY((dispatch_layout<float, 64, 64, 32, 2, 2>(ctx, h, split, vec)));
  else
    TT_TRY((dispatch_layout<float, 128, 128, 32, 2, 2>(ctx, h, split, vec)));
  if (g.colsum && !fused_sum) {
    TT_REQUIRE(ctx, g.epi == EPI_STORE || g.epi == EPI_GELU_BWD, "gemm: column sums of this epilogue");
    return tt_colsum(ctx, g.out_bf16 ? mode : TT_F32, g.M, g.N, g.ldo, g.out, g.colsum);
  }
  return TT_OK;
}
