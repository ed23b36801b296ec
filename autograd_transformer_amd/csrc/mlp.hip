// The tiny classifier's whole training step in one launch.
//
// The tinytorch page (section 8, step 5) trains a two-layer classifier:
// Linear -> GELU -> Linear -> softmax cross-entropy -> backward -> SGD.  At
// its size (tens of rows, a few hundred weights) the step is a few dozen
// kFLOP; run as separate kernels it costs one launch latency per op, so the
// time is launches, not arithmetic.  Here one workgroup keeps the inputs,
// weights and every intermediate in LDS and runs the forward, the fused
// log-softmax cross-entropy (mean over rows), the hand-derived backward and
// the SGD update phase by phase, with a workgroup barrier between phases.
#include <math.h>

#include "tt_internal.h"

namespace {

constexpr int MLP_THREADS = 1024;
constexpr size_t MLP_LDS_FLOATS = 16384;   // 64 KB of dynamic LDS

struct MlpArgs {
  int N, I, H, C;
  const float *x;            // [N, I]
  const int32_t *labels;     // [N]
  float *W1, *b1, *W2, *b2;  // [I, H], [H], [H, C], [C]; updated in place
  float *gW1, *gb1, *gW2, *gb2;   // nullable gradient outputs (written)
  float lr;
  float *loss;               // [1]
  int32_t *range_flag;
};

// Sum over the G consecutive lanes that share one output (G a power of two
// dividing 64): butterfly within the group.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Every phase spreads its outputs over all 1024 threads; the reductions over
// rows (logits, weight gradients) give each output a group of lanes that
// split the rows and meet in a butterfly, so no thread walks a long serial
// chain of LDS reads.
__global__ void __launch_bounds__(MLP_THREADS) mlp_step_kernel(MlpArgs a) {
  extern __shared__ float lds[];
  const int N = a.N, I = a.I, H = a.H, C = a.C, tid = threadIdx.x;
  float *x = lds;                 // N*I
  float *w1 = x + N * I;          // I*H
  float *b1 = w1 + I * H;         // H
  float *w2 = b1 + H;             // H*C
  float *b2 = w2 + H * C;         // C
  float *hp = b2 + C;             // N*H: pre-activation, later its gradient
  float *h = hp + N * H;          // N*H: GELU output
  float *z = h + N * H;           // N*C: logits, later their gradient
  float *rl = z + N * C;          // N: per-row losses
  for (int i = tid; i < N * I; i += MLP_THREADS) x[i] = a.x[i];
  for (int i = tid; i < I * H; i += MLP_THREADS) w1[i] = a.W1[i];
  for (int i = tid; i < H; i += MLP_THREADS) b1[i] = a.b1[i];
  for (int i = tid; i < H * C; i += MLP_THREADS) w2[i] = a.W2[i];
  for (int i = tid; i < C; i += MLP_THREADS) b2[i] = a.b2[i];
  __syncthreads();
  // forward: hp = x W1 + b1, h = GELU(hp)
  for (int e = tid; e < N * H; e += MLP_THREADS) {
    const int n = e / H, j = e - n * H;
    float s = b1[j];
    for (int i = 0; i < I; ++i) s += x[n * I + i] * w1[i * H + j];
    hp[e] = s;
    h[e] = gelu_f(s);
  }
  __syncthreads();
  // z = h W2 + b2: 4 lanes per logit, each over a quarter of the hidden units
  {
    constexpr int G = 4;
    const int sub = tid & (G - 1);
    for (int base = tid - sub; base < N * C * G; base += MLP_THREADS) {
      const int e = base / G;
      float s = 0.f;
      if (e < N * C) {
        const int n = e / C, c = e - n * C;
        for (int j = sub; j < H; j += G) s += h[n * H + j] * w2[j * C + c];
      }
      s = group_sum<G>(s);
      if (sub == 0 && e < N * C) z[e] = s + b2[e % C];
    }
  }
  __syncthreads();
  // cross-entropy per row: loss_n = logsumexp(z_n) - z_n[y_n];
  // dz_n = (softmax(z_n) - onehot(y_n)) / N, written over z.  With
  // e_c = exp(z_c - max) and r = sum of e_c over c != y: the label's entry
  // p_y - 1 = -r / (e_y + r), and the loss is log1p(r / e_y) when the label
  // holds the maximum -- both free of the cancellation of 1 - p_y in float32
  // when a row is predicted confidently.
  const float invN = 1.f / (float)N;
  for (int n = tid; n < N; n += MLP_THREADS) {
    float *zr = z + n * C;
    const int y = a.labels[n];
    const bool ok = y >= 0 && y < C;
    if (!ok) {
      atomicOr(a.range_flag, 1);
      rl[n] = NAN;
      for (int c = 0; c < C; ++c) zr[c] = NAN;
      continue;
    }
    float m = -INFINITY;
    for (int c = 0; c < C; ++c) m = fmaxf(m, zr[c]);
    float r = 0.f;
    for (int c = 0; c < C; ++c)
      if (c != y) r += __expf(zr[c] - m);
    const float ey = __expf(zr[y] - m);
    const float s = ey + r;
    rl[n] = zr[y] == m ? log1pf(r / ey) : m + __logf(s) - zr[y];
    const float inv = invN / s;
    for (int c = 0; c < C; ++c) zr[c] = c == y ? -r * inv : __expf(zr[c] - m) * inv;
  }
  __syncthreads();
  if (tid < 64) {   // mean loss: one wave adds the row losses
    float t = 0.f;
    for (int n = tid; n < N; n += 64) t += rl[n];
    t = wave_sum(t);
    if (tid == 0) *a.loss = t * invN;
  }
  // dW2 = hᵀ dz, db2 = column sums of dz (old W2 still in LDS): 8 lanes per
  // output, each over every 8th row
  {
    constexpr int G = 8;
    const int sub = tid & (G - 1);
    for (int base = tid - sub; base < (H * C + C) * G; base += MLP_THREADS) {
      const int e = base / G;
      float s = 0.f;
      if (e < H * C) {
        const int j = e / C, c = e - j * C;
        for (int n = sub; n < N; n += G) s += h[n * H + j] * z[n * C + c];
      } else if (e < H * C + C) {
        const int c = e - H * C;
        for (int n = sub; n < N; n += G) s += z[n * C + c];
      }
      s = group_sum<G>(s);
      if (sub == 0 && e < H * C) {
        if (a.gW2) a.gW2[e] = s;
        a.W2[e] = w2[e] - a.lr * s;
      } else if (sub == 0 && e < H * C + C) {
        const int c = e - H * C;
        if (a.gb2) a.gb2[c] = s;
        a.b2[c] = b2[c] - a.lr * s;
      }
    }
  }
  // dhp = (dz W2ᵀ) * GELU'(hp), written over hp
  for (int e = tid; e < N * H; e += MLP_THREADS) {
    const int n = e / H, j = e - n * H;
    float s = 0.f;
    for (int c = 0; c < C; ++c) s += z[n * C + c] * w2[j * C + c];
    hp[e] = s * gelu_grad_f(hp[e]);
  }
  __syncthreads();
  // dW1 = xᵀ dhp, db1 = column sums of dhp: 8 lanes per output
  {
    constexpr int G = 8;
    const int sub = tid & (G - 1);
    for (int base = tid - sub; base < (I * H + H) * G; base += MLP_THREADS) {
      const int e = base / G;
      float s = 0.f;
      if (e < I * H) {
        const int i = e / H, j = e - i * H;
        for (int n = sub; n < N; n += G) s += x[n * I + i] * hp[n * H + j];
      } else if (e < I * H + H) {
        const int j = e - I * H;
        for (int n = sub; n < N; n += G) s += hp[n * H + j];
      }
      s = group_sum<G>(s);
      if (sub == 0 && e < I * H) {
        if (a.gW1) a.gW1[e] = s;
        a.W1[e] = w1[e] - a.lr * s;
      } else if (sub == 0 && e < I * H + H) {
        const int j = e - I * H;
        if (a.gb1) a.gb1[j] = s;
        a.b1[j] = b1[j] - a.lr * s;
      }
    }
  }
}

}  // namespace

extern "C" int tt_mlp_step(tt_ctx *ctx, int N, int I, int H, int C, const float *x,
                           const int32_t *labels, float *W1, float *b1, float *W2, float *b2,
                           float lr, float *loss, float *gW1, float *gb1, float *gW2, float *gb2) {
  TT_TRY(tt_check_ctx(ctx));
  TT_REQUIRE(ctx, N > 0 && I > 0 && H > 0 && C > 0, "mlp_step: bad shape");
  TT_REQUIRE(ctx, x && labels && W1 && b1 && W2 && b2 && loss, "mlp_step: NULL operand");
  const size_t floats = (size_t)N * I + (size_t)I * H + H + (size_t)H * C + C +
                        2 * (size_t)N * H + (size_t)N * C + N;
  TT_REQUIRE(ctx, floats <= MLP_LDS_FLOATS,
             "mlp_step: %zu floats of inputs, weights and activations exceed the 64 KB "
             "workgroup budget", floats);
  MlpArgs a{N, I, H, C, x, labels, W1, b1, W2, b2, gW1, gb1, gW2, gb2, lr, loss, ctx->dev_flags};
  const double flops = 2.0 * N * (I * H + H * C) * 3.0;
  tt_prof_scope prof(ctx, "mlp_step_kernel", flops, 4.0 * floats);
  hipLaunchKernelGGL(mlp_step_kernel, dim3(1), dim3(MLP_THREADS), floats * 4, ctx->stream, a);
  return tt_check_launch(ctx, "mlp_step");
}
