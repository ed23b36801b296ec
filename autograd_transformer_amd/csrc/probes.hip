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
