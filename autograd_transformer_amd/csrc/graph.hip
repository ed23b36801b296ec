// Recorded-graph autograd over the library's ops (float32).
//
// The tinytorch page (section 3 item 3) builds the graph while the forward
// code runs: every operation returns a new tensor that remembers its op and
// its inputs, and Backward walks from the loss back to the inputs applying
// each op's gradient rule.  Its own Forward and Backward recurse through the
// inputs; the same page's comparison table names a non-recursive walk in
// topological order as the more efficient form.  Here a node can only take
// inputs created before it, so creation order is a topological order: the
// forward runs the needed nodes front to back, the backward the reachable
// ones back to front, and a node used twice simply receives two `+=`
// contributions (gradients accumulate; the C++/CUDA page, section 3.2, keeps
// them in their own storage).  Every op enqueues the same HIP kernels as the
// op-level entry points (GEMMs, GELU, fused cross-entropy) or the small
// kernels below; nothing runs on the host.
#include <math.h>
#include <string.h>

#include <vector>

#include "tt_internal.h"

#define TT_GRAPH_MAGIC 0x54544752u  // "TTGR"

namespace {

enum GOp { G_LEAF, G_MATMUL, G_ADD, G_GELU, G_SOFTMAX, G_CE };

struct GNode {
  int op;
  int a = -1, b = -1;
  int rows, cols;
  float *val = nullptr;     // [rows, cols]
  float *grad = nullptr;    // [rows, cols] or null when no gradient flows here
  bool needs_grad = false;
  bool bcast = false;       // G_ADD: b is one row added to every row of a
  const int32_t *targets = nullptr;   // G_CE: [rows of the logits]
  float *saved = nullptr;   // G_CE: dlogits of a unit upstream gradient
};

__global__ void add_kernel(int rows, int cols, const float *__restrict__ a,
                           const float *__restrict__ b, int bcast, float *__restrict__ y) {
  const size_t n = (size_t)rows * cols;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = a[i] + b[bcast ? i % cols : i];
}

// dst += s * src, s = *scale when scale is given, else 1.
__global__ void acc_kernel(size_t n, const float *__restrict__ scale, const float *__restrict__ src,
                           float *__restrict__ dst) {
  const float s = scale ? *scale : 1.f;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] += s * src[i];
}

__global__ void copy_kernel(size_t n, const float *__restrict__ src, float *__restrict__ dst) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void gelu_fwd_g_kernel(size_t n, const float *__restrict__ x, float *__restrict__ y) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    y[i] = gelu_f(x[i]);
}

__global__ void gelu_bwd_acc_kernel(size_t n, const float *__restrict__ x,
                                    const float *__restrict__ dy, float *__restrict__ dx) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dx[i] += dy[i] * gelu_grad_f(x[i]);
}

// One wave per row: p = exp(x - max) / sum.
__global__ void __launch_bounds__(256) softmax_rows_kernel(int rows, int cols,
                                                           const float *__restrict__ x,
                                                           float *__restrict__ p) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float *xr = x + (size_t)row * cols;
  float m = -INFINITY;
  for (int c = lane; c < cols; c += 64) m = fmaxf(m, xr[c]);
  m = wave_max(m);
  float s = 0.f;
  for (int c = lane; c < cols; c += 64) s += __expf(xr[c] - m);
  s = wave_sum(s);
  const float inv = 1.f / s;
  for (int c = lane; c < cols; c += 64) p[(size_t)row * cols + c] = __expf(xr[c] - m) * inv;
}

// dx += p * (dp - sum_c dp * p) per row (the softmax Jacobian applied to dp).
__global__ void __launch_bounds__(256) softmax_bwd_acc_kernel(int rows, int cols,
                                                              const float *__restrict__ p,
                                                              const float *__restrict__ dp,
                                                              float *__restrict__ dx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const size_t o = (size_t)row * cols;
  float s = 0.f;
  for (int c = lane; c < cols; c += 64) s += dp[o + c] * p[o + c];
  s = wave_sum(s);
  for (int c = lane; c < cols; c += 64) dx[o + c] += p[o + c] * (dp[o + c] - s);
}

inline int grid_of(size_t n) {
  const size_t g = (n + 255) / 256;
  return (int)(g < 4096 ? (g ? g : 1) : 4096);
}

}  // namespace

struct tt_graph {
  uint32_t magic;
  tt_ctx *ctx;
  std::vector<GNode> nodes;
  // a captured training step (tt_graph_capture_sgd_step)
  hipStream_t cap = nullptr;
  hipGraphExec_t step = nullptr;
};

namespace {

int check_graph(tt_graph *g) {
  if (!g) return TT_EINVAL;
  if (g->magic != TT_GRAPH_MAGIC) return TT_ESTALE;
  return tt_check_ctx(g->ctx);
}

#define GRAPH_ENTRY(g, what)                                                   \
  do {                                                                         \
    int _rc = check_graph(g);                                                  \
    if (_rc != TT_OK) return _rc;                                              \
  } while (0)

bool valid_id(const tt_graph *g, int id) { return id >= 0 && id < (int)g->nodes.size(); }

// Add a computed node of the given shape; its value (and, when a gradient
// flows through it, its gradient) are carved from the arena.
int add_node(tt_graph *g, GNode n, int *id) {
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, id != nullptr, "graph: id output is NULL");
  const size_t bytes = (size_t)n.rows * n.cols * 4;
  void *p;
  TT_TRY(tt_arena_alloc(ctx, bytes, &p));
  n.val = (float *)p;
  if (n.needs_grad) {
    TT_TRY(tt_arena_alloc(ctx, bytes, &p));
    n.grad = (float *)p;
  }
  if (n.op == G_CE) {
    const GNode &z = g->nodes[n.a];
    TT_TRY(tt_arena_alloc(ctx, (size_t)z.rows * z.cols * 4, &p));
    n.saved = (float *)p;
  }
  g->nodes.push_back(n);
  *id = (int)g->nodes.size() - 1;
  return TT_OK;
}

int run_forward(tt_graph *g, int i) {
  tt_ctx *ctx = g->ctx;
  GNode &n = g->nodes[i];
  const size_t cnt = (size_t)n.rows * n.cols;
  switch (n.op) {
    case G_LEAF:
      return TT_OK;
    case G_MATMUL: {
      const GNode &A = g->nodes[n.a], &B = g->nodes[n.b];
      GemmArgs ga;
      memset(&ga, 0, sizeof ga);
      ga.A = A.val; ga.lda = A.cols; ga.a_kmajor = true;
      ga.B = B.val; ga.ldb = B.cols; ga.b_kmajor = false;
      ga.M = A.rows; ga.N = B.cols; ga.K = A.cols;
      ga.epi = EPI_STORE; ga.out = n.val; ga.ldo = n.cols;
      return tt_gemm(ctx, TT_F32, ga);
    }
    case G_ADD: {
      tt_prof_scope prof(ctx, "add_kernel", 0.0, 12.0 * cnt);
      hipLaunchKernelGGL(add_kernel, dim3(grid_of(cnt)), dim3(256), 0, ctx->stream, n.rows, n.cols,
                         g->nodes[n.a].val, g->nodes[n.b].val, (int)n.bcast, n.val);
      return tt_check_launch(ctx, "graph add");
    }
    case G_GELU: {
      tt_prof_scope prof(ctx, "gelu_fwd_g_kernel", 0.0, 8.0 * cnt);
      hipLaunchKernelGGL(gelu_fwd_g_kernel, dim3(grid_of(cnt)), dim3(256), 0, ctx->stream, cnt,
                         g->nodes[n.a].val, n.val);
      return tt_check_launch(ctx, "graph gelu");
    }
    case G_SOFTMAX: {
      tt_prof_scope prof(ctx, "softmax_rows_kernel", 0.0, 8.0 * cnt);
      hipLaunchKernelGGL(softmax_rows_kernel, dim3((n.rows + 3) / 4), dim3(256), 0, ctx->stream,
                         n.rows, n.cols, g->nodes[n.a].val, n.val);
      return tt_check_launch(ctx, "graph softmax");
    }
    case G_CE: {
      // the fused log-softmax cross-entropy leaves dlogits (for a unit
      // upstream gradient, mean over rows) in the node's saved buffer
      const GNode &z = g->nodes[n.a];
      const size_t zc = (size_t)z.rows * z.cols;
      {
        tt_prof_scope prof(ctx, "copy_kernel", 0.0, 8.0 * zc);
        hipLaunchKernelGGL(copy_kernel, dim3(grid_of(zc)), dim3(256), 0, ctx->stream, zc, z.val,
                           n.saved);
        TT_TRY(tt_check_launch(ctx, "graph ce copy"));
      }
      return tt_ce_fwdbwd(ctx, TT_F32, z.rows, z.cols, z.cols, n.saved, n.targets, n.val, 0.f);
    }
  }
  return tt_set_error(ctx, TT_EINVAL, "graph: bad node %d", i);
}

// dst += src (optionally scaled by a device scalar).
int accumulate(tt_ctx *ctx, float *dst, const float *src, size_t n, const float *scale = nullptr) {
  tt_prof_scope prof(ctx, "acc_kernel", 0.0, 12.0 * n);
  hipLaunchKernelGGL(acc_kernel, dim3(grid_of(n)), dim3(256), 0, ctx->stream, n, scale, src, dst);
  return tt_check_launch(ctx, "graph accumulate");
}

// Apply node i's gradient rule: its inputs' gradients += contributions of
// n.grad.
int run_backward(tt_graph *g, int i) {
  tt_ctx *ctx = g->ctx;
  GNode &n = g->nodes[i];
  const size_t cnt = (size_t)n.rows * n.cols;
  switch (n.op) {
    case G_MATMUL: {
      // C = A B: dA += dC Bᵀ, dB += Aᵀ dC (the tinytorch page's MatMul rules)
      GNode &A = g->nodes[n.a], &B = g->nodes[n.b];
      const int M = A.rows, K = A.cols, N = B.cols;
      if (A.needs_grad) {
        GemmArgs ga;
        memset(&ga, 0, sizeof ga);
        ga.A = n.grad; ga.lda = N; ga.a_kmajor = true;
        ga.B = B.val; ga.ldb = N; ga.b_kmajor = true;
        ga.M = M; ga.N = K; ga.K = N;
        ga.epi = EPI_STORE_ACC; ga.out = A.grad; ga.ldo = K;
        TT_TRY(tt_gemm(ctx, TT_F32, ga));
      }
      if (B.needs_grad) {
        GemmArgs ga;
        memset(&ga, 0, sizeof ga);
        ga.A = A.val; ga.lda = K; ga.a_kmajor = false;
        ga.B = n.grad; ga.ldb = N; ga.b_kmajor = false;
        ga.M = K; ga.N = N; ga.K = M;
        ga.epi = EPI_ACCUM; ga.out = B.grad; ga.ldo = N;
        TT_TRY(tt_gemm(ctx, TT_F32, ga));
      }
      return TT_OK;
    }
    case G_ADD: {
      GNode &A = g->nodes[n.a], &B = g->nodes[n.b];
      if (A.needs_grad) TT_TRY(accumulate(ctx, A.grad, n.grad, cnt));
      if (B.needs_grad) {
        if (n.bcast) TT_TRY(tt_colsum(ctx, false, n.rows, n.cols, n.cols, n.grad, B.grad));
        else TT_TRY(accumulate(ctx, B.grad, n.grad, cnt));
      }
      return TT_OK;
    }
    case G_GELU: {
      GNode &A = g->nodes[n.a];
      tt_prof_scope prof(ctx, "gelu_bwd_acc_kernel", 0.0, 16.0 * cnt);
      hipLaunchKernelGGL(gelu_bwd_acc_kernel, dim3(grid_of(cnt)), dim3(256), 0, ctx->stream, cnt,
                         A.val, n.grad, A.grad);
      return tt_check_launch(ctx, "graph gelu bwd");
    }
    case G_SOFTMAX: {
      GNode &A = g->nodes[n.a];
      tt_prof_scope prof(ctx, "softmax_bwd_acc_kernel", 0.0, 16.0 * cnt);
      hipLaunchKernelGGL(softmax_bwd_acc_kernel, dim3((n.rows + 3) / 4), dim3(256), 0, ctx->stream,
                         n.rows, n.cols, n.val, n.grad, A.grad);
      return tt_check_launch(ctx, "graph softmax bwd");
    }
    case G_CE: {
      // dlogits += dloss * (softmax - onehot) / rows
      GNode &Z = g->nodes[n.a];
      return accumulate(ctx, Z.grad, n.saved, (size_t)Z.rows * Z.cols, n.grad);
    }
  }
  return TT_OK;
}

}  // namespace

extern "C" int tt_graph_create(tt_ctx *ctx, tt_graph **out) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, out != nullptr, "graph_create: out is NULL");
  tt_graph *g = new tt_graph();
  g->magic = TT_GRAPH_MAGIC;
  g->ctx = ctx;
  *out = g;
  return TT_OK;
}

extern "C" void tt_graph_destroy(tt_graph *g) {
  if (!g || g->magic != TT_GRAPH_MAGIC) return;
  g->magic = 0;
  if (g->step || g->cap) {
    (void)hipStreamSynchronize(g->ctx->stream);   // a replay may still run
    if (g->step) (void)hipGraphExecDestroy(g->step);
    if (g->cap) (void)hipStreamDestroy(g->cap);
  }
  delete g;
}

extern "C" int tt_graph_leaf(tt_graph *g, int rows, int cols, float *data, float *grad, int *id) {
  GRAPH_ENTRY(g, "leaf");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, rows > 0 && cols > 0 && data && id, "graph_leaf: bad arguments");
  TT_REQUIRE(ctx, tt_aligned16(data) && tt_aligned16(grad), "graph_leaf: 16-byte alignment");
  GNode n;
  n.op = G_LEAF;
  n.rows = rows; n.cols = cols;
  n.val = data; n.grad = grad; n.needs_grad = grad != nullptr;
  g->nodes.push_back(n);
  *id = (int)g->nodes.size() - 1;
  return TT_OK;
}

extern "C" int tt_graph_matmul(tt_graph *g, int a, int b, int *id) {
  GRAPH_ENTRY(g, "matmul");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, valid_id(g, a) && valid_id(g, b), "graph_matmul: bad input id");
  const GNode &A = g->nodes[a], &B = g->nodes[b];
  TT_REQUIRE(ctx, A.cols == B.rows, "graph_matmul: [%d,%d] x [%d,%d]", A.rows, A.cols, B.rows, B.cols);
  GNode n;
  n.op = G_MATMUL; n.a = a; n.b = b;
  n.rows = A.rows; n.cols = B.cols;
  n.needs_grad = A.needs_grad || B.needs_grad;
  return add_node(g, n, id);
}

extern "C" int tt_graph_add(tt_graph *g, int a, int b, int *id) {
  GRAPH_ENTRY(g, "add");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, valid_id(g, a) && valid_id(g, b), "graph_add: bad input id");
  const GNode &A = g->nodes[a], &B = g->nodes[b];
  const bool same = A.rows == B.rows && A.cols == B.cols;
  const bool bcast = !same && B.rows == 1 && B.cols == A.cols;
  TT_REQUIRE(ctx, same || bcast, "graph_add: [%d,%d] + [%d,%d]", A.rows, A.cols, B.rows, B.cols);
  GNode n;
  n.op = G_ADD; n.a = a; n.b = b;
  n.rows = A.rows; n.cols = A.cols; n.bcast = bcast;
  n.needs_grad = A.needs_grad || B.needs_grad;
  return add_node(g, n, id);
}

static int unary(tt_graph *g, int op, int a, int *id, const char *what) {
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, valid_id(g, a), "graph_%s: bad input id", what);
  const GNode &A = g->nodes[a];
  GNode n;
  n.op = op; n.a = a;
  n.rows = A.rows; n.cols = A.cols;
  n.needs_grad = A.needs_grad;
  return add_node(g, n, id);
}

extern "C" int tt_graph_gelu(tt_graph *g, int a, int *id) {
  GRAPH_ENTRY(g, "gelu");
  return unary(g, G_GELU, a, id, "gelu");
}

extern "C" int tt_graph_softmax(tt_graph *g, int a, int *id) {
  GRAPH_ENTRY(g, "softmax");
  return unary(g, G_SOFTMAX, a, id, "softmax");
}

extern "C" int tt_graph_cross_entropy(tt_graph *g, int logits, const int32_t *targets, int *id) {
  GRAPH_ENTRY(g, "cross_entropy");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, valid_id(g, logits) && targets, "graph_cross_entropy: bad arguments");
  GNode n;
  n.op = G_CE; n.a = logits; n.targets = targets;
  n.rows = 1; n.cols = 1;
  n.needs_grad = g->nodes[logits].needs_grad;
  return add_node(g, n, id);
}

extern "C" int tt_graph_forward(tt_graph *g, int node) {
  GRAPH_ENTRY(g, "forward");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, valid_id(g, node), "graph_forward: bad node id");
  // the ancestors of node, found back to front, then run front to back
  std::vector<char> need(node + 1, 0);
  need[node] = 1;
  for (int i = node; i >= 0; --i) {
    if (!need[i]) continue;
    const GNode &n = g->nodes[i];
    if (n.a >= 0) need[n.a] = 1;
    if (n.b >= 0) need[n.b] = 1;
  }
  for (int i = 0; i <= node; ++i)
    if (need[i]) TT_TRY(run_forward(g, i));
  return TT_OK;
}

extern "C" int tt_graph_backward(tt_graph *g, int loss) {
  GRAPH_ENTRY(g, "backward");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, valid_id(g, loss), "graph_backward: bad node id");
  const GNode &L = g->nodes[loss];
  TT_REQUIRE(ctx, L.rows == 1 && L.cols == 1 && L.op != G_LEAF,
             "graph_backward: the loss must be a computed [1,1] node");
  if (!L.needs_grad) return TT_OK;   // nothing upstream wants a gradient
  std::vector<char> reach(loss + 1, 0);
  reach[loss] = 1;
  for (int i = loss; i >= 0; --i) {
    const GNode &n = g->nodes[i];
    if (!reach[i] || !n.needs_grad) continue;
    if (n.a >= 0 && g->nodes[n.a].needs_grad) reach[n.a] = 1;
    if (n.b >= 0 && g->nodes[n.b].needs_grad) reach[n.b] = 1;
  }
  // interior gradients start from zero on every backward; leaf gradients
  // accumulate until tt_graph_zero_grad
  for (int i = 0; i <= loss; ++i) {
    const GNode &n = g->nodes[i];
    if (reach[i] && n.op != G_LEAF)
      TT_TRY(tt_fill_f32(ctx, n.grad, (size_t)n.rows * n.cols, i == loss ? 1.f : 0.f));
  }
  for (int i = loss; i >= 0; --i)
    if (reach[i] && g->nodes[i].op != G_LEAF) TT_TRY(run_backward(g, i));
  return TT_OK;
}

extern "C" int tt_graph_zero_grad(tt_graph *g) {
  GRAPH_ENTRY(g, "zero_grad");
  for (const GNode &n : g->nodes)
    if (n.grad) TT_TRY(tt_fill_f32(g->ctx, n.grad, (size_t)n.rows * n.cols, 0.f));
  return TT_OK;
}

extern "C" int tt_graph_tensor(tt_graph *g, int id, float **value, float **grad, int *rows,
                               int *cols) {
  GRAPH_ENTRY(g, "tensor");
  TT_REQUIRE(g->ctx, valid_id(g, id), "graph_tensor: bad node id");
  const GNode &n = g->nodes[id];
  if (value) *value = n.val;
  if (grad) *grad = n.grad;
  if (rows) *rows = n.rows;
  if (cols) *cols = n.cols;
  return TT_OK;
}

// One SGD training step as a HIP graph: the launches of forward(loss),
// zero_grad, backward(loss) and w -= lr * g on every leaf with a gradient,
// recorded once on a private stream (the context's stream may be one that
// cannot be captured) and replayed by tt_graph_step with one launch.
static int record_sgd_step(tt_graph *g, int loss, float lr) {
  TT_TRY(tt_graph_forward(g, loss));
  TT_TRY(tt_graph_zero_grad(g));
  TT_TRY(tt_graph_backward(g, loss));
  for (const GNode &n : g->nodes)
    if (n.op == G_LEAF && n.grad)
      TT_TRY(tt_sgd_step(g->ctx, n.val, n.grad, (size_t)n.rows * n.cols, lr));
  return TT_OK;
}

extern "C" int tt_graph_capture_sgd_step(tt_graph *g, int loss, float lr) {
  GRAPH_ENTRY(g, "capture_sgd_step");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, valid_id(g, loss), "graph_capture_sgd_step: bad node id");
  TT_REQUIRE(ctx, !ctx->profiling, "graph_capture_sgd_step: not while profiling");
  hipError_t e = hipStreamSynchronize(ctx->stream);
  if (e == hipSuccess && !g->cap) e = hipStreamCreateWithFlags(&g->cap, hipStreamNonBlocking);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "graph capture: %s", hipGetErrorString(e));
  if (g->step) {
    (void)hipGraphExecDestroy(g->step);
    g->step = nullptr;
  }
  hipStream_t user = ctx->stream;
  ctx->stream = g->cap;
  e = hipStreamBeginCapture(g->cap, hipStreamCaptureModeThreadLocal);
  int rc = e == hipSuccess ? record_sgd_step(g, loss, lr)
                           : tt_set_error(ctx, TT_EHIP, "graph capture: %s", hipGetErrorString(e));
  hipGraph_t graph = nullptr;
  if (e == hipSuccess) {
    hipError_t e2 = hipStreamEndCapture(g->cap, &graph);
    if (rc == TT_OK && e2 != hipSuccess)
      rc = tt_set_error(ctx, TT_EHIP, "graph capture end: %s", hipGetErrorString(e2));
  }
  ctx->stream = user;
  if (rc == TT_OK) {
    e = hipGraphInstantiate(&g->step, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
      g->step = nullptr;
      rc = tt_set_error(ctx, TT_EHIP, "graph instantiate: %s", hipGetErrorString(e));
    }
  }
  if (graph) (void)hipGraphDestroy(graph);
  return rc;
}

extern "C" int tt_graph_step(tt_graph *g) {
  GRAPH_ENTRY(g, "step");
  tt_ctx *ctx = g->ctx;
  TT_REQUIRE(ctx, g->step != nullptr, "graph_step: no captured step");
  hipError_t e = hipGraphLaunch(g->step, ctx->stream);
  if (e != hipSuccess) return tt_set_error(ctx, TT_EHIP, "graph_step: %s", hipGetErrorString(e));
  return TT_OK;
}
