// Context, HBM arena and error reporting of libtt.
//
// The arena follows the tinytorch page's TensorContext (section 3 item 1):
// one pre-allocated block, tensors carved by bumping an offset, everything
// after a point freed at once by moving the offset back.  Here the block is
// device memory (one hipMalloc, or caller-owned memory such as a torch
// buffer) and carving is 256-byte aligned.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "tt_internal.h"

extern "C" const char *tt_strerror(int status) {
  switch (status) {
    case TT_OK: return "ok";
    case TT_EINVAL: return "invalid argument";
    case TT_ENOMEM: return "out of memory (arena exhausted or device allocation failed)";
    case TT_EHIP: return "HIP runtime error";
    case TT_ESTALE: return "stale or foreign handle";
    case TT_ENONFINITE: return "non-finite value";
    case TT_EUNSUPPORTED: return "unsupported shape";
    case TT_ERANGE: return "index out of range (token id or target)";
    default: return "unknown status";
  }
}

int tt_check_ctx(const tt_ctx *ctx) {
  if (!ctx) return TT_EINVAL;
  if (ctx->magic != TT_CTX_MAGIC) return TT_ESTALE;
  return TT_OK;
}

int tt_set_error(tt_ctx *ctx, int status, const char *fmt, ...) {
  if (ctx && ctx->magic == TT_CTX_MAGIC) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    ctx->last_error = buf;
  }
  return status;
}

int tt_check_launch(tt_ctx *ctx, const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return tt_set_error(ctx, TT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return TT_OK;
}

int tt_arena_alloc(tt_ctx *ctx, size_t bytes, void **p) {
  size_t off = (ctx->offset + 255) & ~(size_t)255;
  if (off > ctx->capacity || bytes > ctx->capacity - off)
    return tt_set_error(ctx, TT_ENOMEM, "arena exhausted: need %zu bytes at offset %zu of %zu",
                        bytes, off, ctx->capacity);
  *p = ctx->arena + off;
  ctx->offset = off + bytes;
  return TT_OK;
}

extern "C" int tt_ctx_create(int device, void *hip_stream, size_t arena_bytes, void *arena_base,
                             tt_ctx **out) {
  if (!out) return TT_EINVAL;
  *out = nullptr;
  if (arena_bytes < 4096) return TT_EINVAL;
  if (arena_base && !tt_aligned16(arena_base)) return TT_EINVAL;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess) return TT_EHIP;
  if (device < 0 || device >= ndev) return TT_EINVAL;
  if (hipSetDevice(device) != hipSuccess) return TT_EHIP;
  tt_ctx *c = new tt_ctx();
  c->magic = TT_CTX_MAGIC;
  c->device = device;
  c->stream = (hipStream_t)hip_stream;
  c->capacity = arena_bytes;
  c->offset = 0;
  c->mark = 0;
  c->owns_arena = arena_base == nullptr;
  c->dev_flags = nullptr;
  if (arena_base) {
    c->arena = (char *)arena_base;
  } else {
    void *p = nullptr;
    if (hipMalloc(&p, arena_bytes) != hipSuccess) {
      (void)hipGetLastError();
      delete c;
      return TT_ENOMEM;
    }
    c->arena = (char *)p;
  }
  if (hipMalloc((void **)&c->dev_flags, 256) != hipSuccess ||
      hipMemset(c->dev_flags, 0, 256) != hipSuccess) {
    (void)hipGetLastError();
    if (c->owns_arena) (void)hipFree(c->arena);
    delete c;
    return TT_ENOMEM;
  }
  // the fixed workspace of tt_layernorm_bwd_noalloc on this device (looked
  // up once per device, with the device current)
  const int rc = tt_noalloc_init(device);
  if (rc != TT_OK) {
    (void)hipFree(c->dev_flags);
    if (c->owns_arena) (void)hipFree(c->arena);
    delete c;
    return rc;
  }
  *out = c;
  return TT_OK;
}

extern "C" void tt_ctx_destroy(tt_ctx *ctx) {
  if (!ctx || ctx->magic != TT_CTX_MAGIC) return;
  (void)hipSetDevice(ctx->device);
  (void)hipStreamSynchronize(ctx->stream);
  for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);
  if (ctx->owns_arena && ctx->arena) (void)hipFree(ctx->arena);
  if (ctx->dev_flags) (void)hipFree(ctx->dev_flags);
  ctx->magic = 0;
  delete ctx;
}

extern "C" int tt_ctx_set_stream(tt_ctx *ctx, void *hip_stream) {
  TT_TRY(tt_check_ctx(ctx));
  ctx->stream = (hipStream_t)hip_stream;
  return TT_OK;
}

extern "C" int tt_ctx_alloc(tt_ctx *ctx, size_t bytes, size_t align, void **dptr) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, dptr != nullptr, "tt_ctx_alloc: dptr is NULL");
  TT_REQUIRE(ctx, align == 0 || (align & (align - 1)) == 0, "tt_ctx_alloc: align not a power of two");
  if (align > 256) {
    size_t off = (ctx->offset + align - 1) & ~(align - 1);
    if (off > ctx->capacity) return tt_set_error(ctx, TT_ENOMEM, "arena exhausted");
    ctx->offset = off;
  }
  return tt_arena_alloc(ctx, bytes, dptr);
}

extern "C" int tt_ctx_mark(tt_ctx *ctx) {
  TT_TRY(tt_check_ctx(ctx));
  ctx->mark = ctx->offset;
  return TT_OK;
}

extern "C" int tt_ctx_reset(tt_ctx *ctx) {
  TT_TRY(tt_check_ctx(ctx));
  ctx->offset = ctx->mark;
  return TT_OK;
}

extern "C" int tt_ctx_usage(const tt_ctx *ctx, size_t *used, size_t *capacity) {
  TT_TRY(tt_check_ctx(ctx));
  if (used) *used = ctx->offset;
  if (capacity) *capacity = ctx->capacity;
  return TT_OK;
}

extern "C" int tt_ctx_sync(tt_ctx *ctx) {
  TT_TRY(tt_check_ctx(ctx));
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "stream: %s", hipGetErrorString(e));
  int32_t flags[4] = {0, 0, 0, 0};
  e = hipMemcpy(flags, ctx->dev_flags, sizeof flags, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "flags: %s", hipGetErrorString(e));
  if (flags[0]) {
    (void)hipMemset(ctx->dev_flags, 0, 16);
    return tt_set_error(ctx, TT_ERANGE, "a token id or target was outside [0, V)");
  }
  return TT_OK;
}

static hipEvent_t prof_event(tt_ctx *ctx) {
  if (ctx->ev_used == ctx->ev_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    ctx->ev_pool.push_back(e);
  }
  return ctx->ev_pool[ctx->ev_used++];
}

tt_prof_scope::tt_prof_scope(tt_ctx *c, const char *name, double flops, double bytes) : ctx(c) {
  if (!ctx->profiling) return;
  tt_prof_rec r{name, flops, bytes, prof_event(ctx), prof_event(ctx)};
  if (!r.e0 || !r.e1) return;
  (void)hipEventRecord(r.e0, ctx->stream);
  idx = (long)ctx->prof.size();
  ctx->prof.push_back(r);
}

tt_prof_scope::~tt_prof_scope() {
  if (idx >= 0) (void)hipEventRecord(ctx->prof[idx].e1, ctx->stream);
}

extern "C" int tt_ctx_profile(tt_ctx *ctx, int enable) {
  TT_TRY(tt_check_ctx(ctx));
  if (enable) {
    ctx->prof.clear();
    ctx->ev_used = 0;
  }
  ctx->profiling = enable != 0;
  return TT_OK;
}

extern "C" int tt_ctx_profile_report(tt_ctx *ctx, tt_prof_entry *out, int *count) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, count != nullptr, "profile_report: count is NULL");
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "profile_report: %s", hipGetErrorString(e));
  std::vector<tt_prof_entry> agg;
  for (const tt_prof_rec &r : ctx->prof) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) {
      (void)hipGetLastError();
      continue;
    }
    size_t i = 0;
    while (i < agg.size() && strcmp(agg[i].name, r.name) != 0) ++i;
    if (i == agg.size()) agg.push_back(tt_prof_entry{r.name, 0, 0.0, 0.0, 0.0});
    agg[i].calls += 1;
    agg[i].ms += ms;
    agg[i].flops += r.flops;
    agg[i].bytes += r.bytes;
  }
  if (out) {
    const int n = (int)agg.size() < *count ? (int)agg.size() : *count;
    for (int i = 0; i < n; ++i) out[i] = agg[i];
  }
  *count = (int)agg.size();
  return TT_OK;
}

extern "C" const char *tt_ctx_last_error(const tt_ctx *ctx) {
  if (!ctx || ctx->magic != TT_CTX_MAGIC) return "invalid context";
  return ctx->last_error.c_str();
}
