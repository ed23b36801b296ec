// LayerNorm backward with its workspace in a fixed device array, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// tt_layernorm_bwd forms the column sums behind dg and db per workgroup into
// a partial-sum workspace carved from the context's arena, then adds them up
// in a second launch.  tt_layernorm_bwd_noalloc runs the same two kernels
// with that workspace in `scratch`, a file-scope device array of
// TT_NOALLOC_SCRATCH_BYTES: every GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (in host code it names a host-side stand-in, not device memory):
// tt_noalloc_init, called by tt_ctx_create with the device current, looks up
// that device's copy once with hipGetSymbolAddress and keeps the address.
#include <mutex>

#include "tt_internal.h"

static __device__ __align__(256) float scratch[TT_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int TT_MAX_DEVICES = 64;

std::mutex g_mu;
void *g_scratch[TT_MAX_DEVICES];   // device address of `scratch` on each device (or null)

}  // namespace

int tt_noalloc_init(int device) {
  if (device < 0 || device >= TT_MAX_DEVICES) return TT_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[device]) return TT_OK;
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return TT_EHIP;
  }
  g_scratch[device] = ptr;
  return TT_OK;
}

extern "C" int tt_layernorm_bwd_noalloc(tt_ctx *ctx, tt_mode mode, int N, int C, const float *x,
                                        const float *mean, const float *rstd, const float *g,
                                        const float *dy, float *dx, float *dg, float *db) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, mode == TT_F32 || mode == TT_BF16 || mode == TT_FP16,
             "layernorm_bwd_noalloc: bad mode");
  TT_REQUIRE(ctx, N >= 0 && C > 0 && C % 4 == 0 && C <= 4096,
             "layernorm_bwd_noalloc: need C %% 4 == 0, C <= 4096");
  TT_REQUIRE(ctx, x && mean && rstd && g && dy && dx, "layernorm_bwd_noalloc: NULL pointer");
  TT_REQUIRE(ctx, tt_aligned16(x) && tt_aligned16(dy) && tt_aligned16(dx) && tt_aligned16(g),
             "layernorm_bwd_noalloc: alignment");
  if (N == 0) return TT_OK;
  const size_t per_group = (size_t)3 * C * sizeof(float);
  const int G = tt_layernorm_bwd_groups(N, C);
  if ((size_t)G * per_group > TT_NOALLOC_SCRATCH_BYTES)
    return tt_set_error(ctx, TT_EINVAL,
                        "layernorm_bwd_noalloc: %d rows of width %d need %zu bytes of workspace, "
                        "above the fixed %zu (use tt_layernorm_bwd)",
                        N, C, (size_t)G * per_group, (size_t)TT_NOALLOC_SCRATCH_BYTES);
  void *ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (ctx->device >= 0 && ctx->device < TT_MAX_DEVICES) ptr = g_scratch[ctx->device];
  }
  if (!ptr)
    return tt_set_error(ctx, TT_EHIP, "layernorm_bwd_noalloc: no workspace on device %d",
                        ctx->device);
  // The kernel timer creates its events on demand: these launches are not
  // timed, so that nothing is created here.
  const bool prof = ctx->profiling;
  ctx->profiling = false;
  const int rc = tt_layernorm_bwd_ws(ctx, mode, N, C, x, mean, rstd, g, dy, dx, dx, nullptr, dg,
                                     db, nullptr, (float *)ptr,
                                     (int)(TT_NOALLOC_SCRATCH_BYTES / per_group));
  ctx->profiling = prof;
  return rc;
}
