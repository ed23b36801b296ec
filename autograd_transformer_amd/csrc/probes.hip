// Roofline probes: what this GPU sustains with nothing else in the way, the
// denominators the measured kernels are held against next to the vendor's
// figures (the C++/CUDA page, section 2.2, times each op with an event pair;
// these time the two ceilings the same way).
//
//  * MFMA: every wave of a full grid issues v_mfma_f32_16x16x32_bf16 on
//    register operands only, over ACC independent accumulators (so no MFMA
//    waits for the previous one), no memory traffic in the loop.
//  * HBM: a streaming read (every 16-byte vector of a buffer far larger than
//    the caches read once, combined so the compiler keeps the loads) and a
//    streaming copy (read once, written once).
//  * Per-CU ceilings, in shader clocks (clock64() around each wave's loop,
//    so the figures do not depend on the clock the part runs at): LDS
//    fragment reads (ds_read_b128) alone and feeding MFMAs, global-to-LDS
//    loads (buffer_load_dwordx4 ... lds) from L2 and from HBM, and the issue
//    cost of VALU, transcendental and MFMA instructions with one or two waves
//    per SIMD, alone and side by side.
#include <algorithm>

#include "tt_internal.h"

namespace {

template <int ACC>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float *__restrict__ out) {
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (threadIdx.x - i));
  }
  // distinct starting values: identical accumulators would let the compiler
  // merge their chains
  f32x4_t acc[ACC];
  const float t = 1e-3f * threadIdx.x;
#pragma unroll
  for (int j = 0; j < ACC; ++j) acc[j] = f32x4_t{t + j, t - j, t * j, t + 2.f * j};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < ACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < ACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  // one store per wave keeps the chain live; the value is never read
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

__global__ void __launch_bounds__(256) read_probe_kernel(size_t n4, const float4 *__restrict__ src,
                                                         float *__restrict__ out) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
    acc += __builtin_nontemporal_load((const v4f *)src + i);
  const float s = acc[0] + acc[1] + acc[2] + acc[3];
  if (s == 1234.5f) out[blockIdx.x] = s;   // practically never: keeps the loads
}

__global__ void __launch_bounds__(256) copy_probe_kernel(size_t n4, const float4 *__restrict__ src,
                                                         float4 *__restrict__ dst) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load((const v4f *)src + i), (v4f *)dst + i);
}

// One workgroup of 8 waves per CU (two per SIMD).  Each iteration a wave
// reads 8 fragments of 1 KB (lane-linear, no bank conflicts) from one of four
// 16 KB LDS slots and, with MFMA, issues the 16 products of a 64 x 64 tile
// on them.  cyc[wave] receives the wave's loop cycles.
template <bool MFMA>
__global__ void __launch_bounds__(512, 1) lds_probe_kernel(int iters, long long *__restrict__ cyc,
                                                           float *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid * 16; i < 65536; i += 512 * 16)
    *(float4 *)(lds + i) = make_float4(1e-3f * i, 1.f, 2.f, 3.f);
  __syncthreads();
  f32x4_t acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, (float)i, (float)j, 1.f};
  uint4 x = make_uint4(0, 0, 0, 0);
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
    const int base = (it & 3) * 16384 + lane * 16;
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *(const bf16x8_t *)(lds + base + i * 1024);
      b[i] = *(const bf16x8_t *)(lds + base + (4 + i) * 1024);
    }
    if constexpr (MFMA) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = __builtin_bit_cast(uint4, a[i]), v = __builtin_bit_cast(uint4, b[i]);
        x.x ^= u.x ^ v.x; x.y ^= u.y ^ v.y; x.z ^= u.z ^ v.z; x.w ^= u.w ^ v.w;
      }
    }
  }
  const long long t1 = clock64();
  float sum = (float)(x.x ^ x.y ^ x.z ^ x.w);
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) sum += acc[i][j][0] + acc[i][j][3];
  if (lane == 0) {
    cyc[blockIdx.x * 8 + (tid >> 6)] = t1 - t0;
    out[blockIdx.x * 8 + (tid >> 6)] = sum;
  }
}

// 8 waves per CU stream a window of `win` bytes of src (workgroup b at
// offset b * win, wrapping inside the buffer) into LDS with 16-byte
// direct-to-LDS loads, 16 in flight per wave.
__global__ void __launch_bounds__(512, 1) lds_load_probe_kernel(const char *__restrict__ src,
                                                                uint32_t bytes, uint32_t win,
                                                                int iters,
                                                                long long *__restrict__ cyc,
                                                                float *__restrict__ out) {
  __shared__ __attribute__((aligned(16))) char lds[65536];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void *)src, (short)0, (int)bytes, 0x00020000);
  const uint32_t base = (uint32_t)(((unsigned long long)blockIdx.x * win) % (bytes - win + 1)) & ~1023u;
  uint32_t pos = (uint32_t)wave * 1024;
  const long long t0 = clock64();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint32_t off = base + ((pos + u * 8192) % win) + lane * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(lds + ((wave * 16 + u) % 64) * 1024), 16,
          off, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    pos = (pos + 16 * 8192) % win;
  }
  const long long t1 = clock64();
  __syncthreads();
  const float v = *(const float *)(lds + tid * 4);
  if (lane == 0) {
    cyc[blockIdx.x * 8 + wave] = t1 - t0;
    if (v == 1234.5f) out[blockIdx.x] = v;   // practically never: keeps the loads
  }
}

// Issue cost per instruction: 8 independent chains per wave of v_fma_f32,
// v_exp_f32 or v_mfma_f32_16x16x32_bf16.  Waves 0-3 (one per SIMD) run role
// R0, waves 4-7 (the second wave of each SIMD) run R1 (0: idle, 1: FMA, 2:
// exp, 3: MFMA).  cyc[wave] receives the wave's loop cycles (0 if idle).
template <int R0, int R1>
__global__ void __launch_bounds__(512, 1) issue_probe_kernel(int iters, long long *__restrict__ cyc,
                                                             float *__restrict__ out) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int role = wave < 4 ? R0 : R1;
  float x[8];
  for (int j = 0; j < 8; ++j) x[j] = 1e-3f * (tid + j) - 0.25f;
  f32x4_t acc[8];
  for (int j = 0; j < 8; ++j) acc[j] = f32x4_t{x[j], 1.f, 2.f, 3.f};
  bf16x8_t a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (tid + i));
    b[i] = (__bf16)(0.002f * (tid - i));
  }
  const long long t0 = clock64();
  if (role == 1) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = fmaf(x[j], 1.0001f, 0.5f);
  } else if (role == 2) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
  } else if (role == 3) {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  const long long t1 = clock64();
  float sum = 0.f;
  for (int j = 0; j < 8; ++j) sum += x[j] + acc[j][0];
  if ((tid & 63) == 0) {
    cyc[blockIdx.x * 8 + wave] = role ? t1 - t0 : 0;
    out[blockIdx.x * 8 + wave] = sum;
  }
}

int elapsed(tt_ctx *ctx, hipEvent_t e0, hipEvent_t e1, double *ms) {
  float f = 0.f;
  hipError_t e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&f, e0, e1);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "probe timing: %s", hipGetErrorString(e));
  *ms = f;
  return TT_OK;
}

struct Events {
  hipEvent_t a = nullptr, b = nullptr;
  ~Events() {
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
  }
};

}  // namespace

extern "C" int tt_probe_mfma(tt_ctx *ctx, int waves_per_simd, int accumulators, int iters,
                             double *tflops) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, tflops && iters > 0 && iters <= (1 << 24), "probe_mfma: bad arguments");
  TT_REQUIRE(ctx, waves_per_simd >= 1 && waves_per_simd <= 8, "probe_mfma: 1..8 waves per SIMD");
  TT_REQUIRE(ctx, accumulators == 8 || accumulators == 16 || accumulators == 32,
             "probe_mfma: 8, 16 or 32 accumulators");
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, ctx->device) != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "probe_mfma: device properties");
  // 4-wave workgroups: one wave per SIMD each, waves_per_simd of them per CU
  const int blocks = prop.multiProcessorCount * waves_per_simd;
  tt_scratch_scope scope(ctx);
  void *out;
  TT_TRY(tt_arena_alloc(ctx, (size_t)blocks * 4 * sizeof(float), &out));
  Events ev;
  if (hipEventCreate(&ev.a) != hipSuccess || hipEventCreate(&ev.b) != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "probe_mfma: events");
  auto launch = [&](int n) {
    if (accumulators == 8)
      hipLaunchKernelGGL(mfma_probe_kernel<8>, dim3(blocks), dim3(256), 0, ctx->stream, n, (float *)out);
    else if (accumulators == 16)
      hipLaunchKernelGGL(mfma_probe_kernel<16>, dim3(blocks), dim3(256), 0, ctx->stream, n, (float *)out);
    else
      hipLaunchKernelGGL(mfma_probe_kernel<32>, dim3(blocks), dim3(256), 0, ctx->stream, n, (float *)out);
  };
  launch(16);   // warm-up (clocks, code)
  TT_TRY(tt_check_launch(ctx, "probe_mfma"));
  (void)hipEventRecord(ev.a, ctx->stream);
  launch(iters);
  (void)hipEventRecord(ev.b, ctx->stream);
  TT_TRY(tt_check_launch(ctx, "probe_mfma"));
  double ms = 0;
  TT_TRY(elapsed(ctx, ev.a, ev.b, &ms));
  const double flops = (double)blocks * 4 * iters * accumulators * 16.0 * 16.0 * 32.0 * 2.0;
  *tflops = flops / (ms * 1e-3) / 1e12;
  return TT_OK;
}

extern "C" int tt_probe_hbm(tt_ctx *ctx, void *buf, size_t bytes, int copy, double *gbs) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, buf && gbs && tt_aligned16(buf), "probe_hbm: bad arguments");
  TT_REQUIRE(ctx, bytes >= (1u << 20) && bytes % 32 == 0, "probe_hbm: at least 1 MiB, multiple of 32");
  const size_t half = bytes / 2;
  const size_t n4 = (copy ? half : bytes) / 16;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, ctx->device) != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "probe_hbm: device properties");
  const int blocks = prop.multiProcessorCount * 8;
  tt_scratch_scope scope(ctx);
  void *out;
  TT_TRY(tt_arena_alloc(ctx, (size_t)blocks * sizeof(float), &out));
  Events ev;
  if (hipEventCreate(&ev.a) != hipSuccess || hipEventCreate(&ev.b) != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "probe_hbm: events");
  auto launch = [&]() {
    if (copy)
      hipLaunchKernelGGL(copy_probe_kernel, dim3(blocks), dim3(256), 0, ctx->stream, n4,
                         (const float4 *)buf, (float4 *)((char *)buf + half));
    else
      hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, ctx->stream, n4,
                         (const float4 *)buf, (float *)out);
  };
  launch();   // warm-up
  TT_TRY(tt_check_launch(ctx, "probe_hbm"));
  (void)hipEventRecord(ev.a, ctx->stream);
  for (int r = 0; r < 5; ++r) launch();
  (void)hipEventRecord(ev.b, ctx->stream);
  TT_TRY(tt_check_launch(ctx, "probe_hbm"));
  double ms = 0;
  TT_TRY(elapsed(ctx, ev.a, ev.b, &ms));
  const double moved = 5.0 * (copy ? 2.0 * half : (double)bytes);
  *gbs = moved / (ms * 1e-3) / 1e9;
  return TT_OK;
}

namespace {

// Mean over workgroups of the slowest wave's cycles among waves [w0, w1).
int mean_max_cycles(tt_ctx *ctx, const long long *dcyc, int blocks, int w0, int w1, double *out) {
  std::vector<long long> h((size_t)blocks * 8);
  hipError_t e = hipMemcpyAsync(h.data(), dcyc, h.size() * sizeof(long long), hipMemcpyDeviceToHost,
                                ctx->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "probe: %s", hipGetErrorString(e));
  double s = 0;
  for (int b = 0; b < blocks; ++b) {
    long long m = 0;
    for (int w = w0; w < w1; ++w) m = std::max(m, h[(size_t)b * 8 + w]);
    s += (double)m;
  }
  *out = s / blocks;
  return TT_OK;
}

int cus_of(tt_ctx *ctx, int *cus) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, ctx->device) != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "probe: device properties");
  *cus = prop.multiProcessorCount;
  return TT_OK;
}

}  // namespace

extern "C" int tt_probe_lds(tt_ctx *ctx, int mfma, double *bytes_per_clk, double *tflops) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, bytes_per_clk && tflops, "probe_lds: NULL output");
  int cus = 0;
  TT_TRY(cus_of(ctx, &cus));
  tt_scratch_scope scope(ctx);
  void *cyc, *out;
  TT_TRY(tt_arena_alloc(ctx, (size_t)cus * 8 * sizeof(long long), &cyc));
  TT_TRY(tt_arena_alloc(ctx, (size_t)cus * 8 * sizeof(float), &out));
  Events ev;
  if (hipEventCreate(&ev.a) != hipSuccess || hipEventCreate(&ev.b) != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "probe_lds: events");
  const int iters = 20000;
  auto launch = [&](int n) {
    if (mfma)
      hipLaunchKernelGGL(lds_probe_kernel<true>, dim3(cus), dim3(512), 0, ctx->stream, n,
                         (long long *)cyc, (float *)out);
    else
      hipLaunchKernelGGL(lds_probe_kernel<false>, dim3(cus), dim3(512), 0, ctx->stream, n,
                         (long long *)cyc, (float *)out);
  };
  launch(100);
  TT_TRY(tt_check_launch(ctx, "probe_lds"));
  (void)hipEventRecord(ev.a, ctx->stream);
  launch(iters);
  (void)hipEventRecord(ev.b, ctx->stream);
  TT_TRY(tt_check_launch(ctx, "probe_lds"));
  double ms = 0, cycles = 0;
  TT_TRY(elapsed(ctx, ev.a, ev.b, &ms));
  TT_TRY(mean_max_cycles(ctx, (const long long *)cyc, cus, 0, 8, &cycles));
  *bytes_per_clk = 8.0 * iters * 8 * 1024 / cycles;
  *tflops = mfma ? (double)cus * 8 * iters * 16 * 16.0 * 16 * 32 * 2 / (ms * 1e-3) / 1e12 : 0.0;
  return TT_OK;
}

extern "C" int tt_probe_lds_load(tt_ctx *ctx, void *buf, size_t bytes, int resident,
                                 double *bytes_per_clk) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, buf && bytes_per_clk && tt_aligned16(buf), "probe_lds_load: bad arguments");
  TT_REQUIRE(ctx, bytes >= ((size_t)64 << 20) && bytes < ((size_t)1 << 31),
             "probe_lds_load: 64 MiB .. 2 GiB buffer");
  int cus = 0;
  TT_TRY(cus_of(ctx, &cus));
  tt_scratch_scope scope(ctx);
  void *cyc, *out;
  TT_TRY(tt_arena_alloc(ctx, (size_t)cus * 8 * sizeof(long long), &cyc));
  TT_TRY(tt_arena_alloc(ctx, (size_t)cus * sizeof(float), &out));
  // L2-resident: 64 KB per workgroup (32 per XCD: 2 MB of its 4 MB L2);
  // streaming: 4 MB per workgroup, the windows tiling the buffer
  const uint32_t win = resident ? 65536u : (4u << 20);
  const int iters = resident ? 4000 : 1000;
  hipLaunchKernelGGL(lds_load_probe_kernel, dim3(cus), dim3(512), 0, ctx->stream, (const char *)buf,
                     (uint32_t)bytes, win, 10, (long long *)cyc, (float *)out);
  hipLaunchKernelGGL(lds_load_probe_kernel, dim3(cus), dim3(512), 0, ctx->stream, (const char *)buf,
                     (uint32_t)bytes, win, iters, (long long *)cyc, (float *)out);
  TT_TRY(tt_check_launch(ctx, "probe_lds_load"));
  double cycles = 0;
  TT_TRY(mean_max_cycles(ctx, (const long long *)cyc, cus, 0, 8, &cycles));
  *bytes_per_clk = 8.0 * iters * 16 * 1024 / cycles;
  return TT_OK;
}

extern "C" int tt_probe_issue(tt_ctx *ctx, int which, double *first, double *second) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, first && second && which >= 0 && which <= 7, "probe_issue: which in 0..7");
  int cus = 0;
  TT_TRY(cus_of(ctx, &cus));
  tt_scratch_scope scope(ctx);
  void *cyc, *out;
  TT_TRY(tt_arena_alloc(ctx, (size_t)cus * 8 * sizeof(long long), &cyc));
  TT_TRY(tt_arena_alloc(ctx, (size_t)cus * 8 * sizeof(float), &out));
  const int iters = 20000;
  auto launch = [&](int n) {
    long long *c = (long long *)cyc;
    float *o = (float *)out;
    switch (which) {
      case 0: hipLaunchKernelGGL((issue_probe_kernel<1, 0>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
      case 1: hipLaunchKernelGGL((issue_probe_kernel<1, 1>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
      case 2: hipLaunchKernelGGL((issue_probe_kernel<2, 0>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
      case 3: hipLaunchKernelGGL((issue_probe_kernel<2, 2>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
      case 4: hipLaunchKernelGGL((issue_probe_kernel<3, 0>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
      case 5: hipLaunchKernelGGL((issue_probe_kernel<3, 3>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
      case 6: hipLaunchKernelGGL((issue_probe_kernel<3, 1>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
      default: hipLaunchKernelGGL((issue_probe_kernel<3, 2>), dim3(cus), dim3(512), 0, ctx->stream, n, c, o); break;
    }
  };
  launch(100);
  launch(iters);
  TT_TRY(tt_check_launch(ctx, "probe_issue"));
  // the first wave of each SIMD (waves 0-3) and the second (waves 4-7; the
  // older wave wins the issue arbitration, so with two busy waves the first
  // finishes early and the second's time is the pair's)
  double c0 = 0, c1 = 0;
  TT_TRY(mean_max_cycles(ctx, (const long long *)cyc, cus, 0, 4, &c0));
  TT_TRY(mean_max_cycles(ctx, (const long long *)cyc, cus, 4, 8, &c1));
  *first = c0 / (8.0 * iters);
  *second = c1 / (8.0 * iters);
  return TT_OK;
}
