"""Per-op forward and hand-derived backward rules, NumPy float64 (test infrastructure only).

Every function is the plain definition of the op written out, with
``numpy.matmul`` as the only library primitive.  Nothing is blocked, fused or
reordered beyond what the definition states.  Conventions:

* Row-major arrays; a linear layer is ``y = x @ W + b`` with ``W`` of shape
  ``[in, out]`` (the tinytorch page's MatMul: ``C[M,N] = A[M,K] @ B[K,N]``).
* Backward functions *return* gradients; accumulation (``+=`` into a shared
  buffer) is done by the caller, as the tinytorch page's MatMul backward note
  prescribes for tensors with several consumers.
* ``store`` arguments are optional callables applied to a tensor at the point
  where it is written to memory (identity for fp32 mode, bf16 rounding for the
  bf16 mode); they model storage precision only, never a change of formula.
"""

import math

import numpy as np


def _ident(a):
    return a


# --------------------------------------------------------------------------
# Linear / MatMul — tinytorch page, section 3 item 3 (MatMulForward /
# MatMulBackward); define-by-run page section 3.2 (dA = dC·Bᵀ, dB = Aᵀ·dC).
# --------------------------------------------------------------------------

def linear_fwd(x, W, b=None):
    """y = x @ W (+ b).  x [M,K], W [K,N], b [N] -> y [M,N]."""
    y = np.matmul(np.asarray(x, np.float64), np.asarray(W, np.float64))
    if b is not None:
        y = y + np.asarray(b, np.float64)[None, :]
    return y


def linear_bwd(x, W, dy, with_bias=True):
    """Gradients of y = x @ W + b.

    dx = dy @ Wᵀ ; dW = xᵀ @ dy ; db = column sums of dy.
    Returns (dx, dW, db) (db is None when ``with_bias`` is False).
    """
    x = np.asarray(x, np.float64)
    W = np.asarray(W, np.float64)
    dy = np.asarray(dy, np.float64)
    dx = np.matmul(dy, W.T)
    dW = np.matmul(x.T, dy)
    db = dy.sum(axis=0) if with_bias else None
    return dx, dW, db


# --------------------------------------------------------------------------
# LayerNorm — tinytorch page section 4 (knowledge table: subtract the mean,
# divide by the standard deviation, scale by the weight, add the bias); Forge
# page "最硬的一关" names epsilon placement and the variance method as the
# pitfalls.  Reading: biased variance mean((x-mu)^2), eps inside the sqrt.
# --------------------------------------------------------------------------

def layernorm_fwd(x, gamma, beta, eps=1e-5):
    """Row-wise LayerNorm over the last axis.

    Returns (y, mean, rstd) with mean, rstd of shape x.shape[:-1].
    """
    x = np.asarray(x, np.float64)
    mean = x.mean(axis=-1)
    xc = x - mean[..., None]
    var = (xc * xc).mean(axis=-1)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = xc * rstd[..., None]
    y = xhat * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)
    return y, mean, rstd


def layernorm_bwd(x, mean, rstd, gamma, dy):
    """Chain rule through y = xhat*gamma + beta, xhat = (x-mean)*rstd.

    With g = dy*gamma (per element) and C the row length:
      dx = rstd * (g - mean_row(g) - xhat * mean_row(g*xhat))
      dgamma = sum over rows of dy*xhat ; dbeta = sum over rows of dy.
    Returns (dx, dgamma, dbeta).
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    gamma = np.asarray(gamma, np.float64)
    xhat = (x - mean[..., None]) * rstd[..., None]
    g = dy * gamma
    mg = g.mean(axis=-1, keepdims=True)
    mgx = (g * xhat).mean(axis=-1, keepdims=True)
    dx = rstd[..., None] * (g - mg - xhat * mgx)
    red = tuple(range(x.ndim - 1))
    dgamma = (dy * xhat).sum(axis=red)
    dbeta = dy.sum(axis=red)
    return dx, dgamma, dbeta


# --------------------------------------------------------------------------
# GELU, tanh form — tinytorch page section 3 item 4:
#   GELU(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).
# The page's backward (cdf = out/x plus x times the exact normal pdf) is not
# the derivative of that forward and is 0/0 at x = 0; the reading used here is
# the analytic derivative of the tanh form, the one central differences
# (define-by-run page section 4.2) confirm.
# --------------------------------------------------------------------------

_GELU_K = math.sqrt(2.0 / math.pi)
_GELU_A = 0.044715


def gelu_fwd(x):
    x = np.asarray(x, np.float64)
    return 0.5 * x * (1.0 + np.tanh(_GELU_K * (x + _GELU_A * x ** 3)))


def gelu_grad(x):
    """d GELU / dx for the tanh form."""
    x = np.asarray(x, np.float64)
    u = _GELU_K * (x + _GELU_A * x ** 3)
    t = np.tanh(u)
    du = _GELU_K * (1.0 + 3.0 * _GELU_A * x * x)
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du


def gelu_bwd(x, dy):
    return np.asarray(dy, np.float64) * gelu_grad(x)


# --------------------------------------------------------------------------
# Softmax and cross-entropy — tinytorch page section 3 item 5 (probs minus the
# one-hot target) and section 4 (subtract the row max before exp); Forge page
# "核心组件清单" (cross-entropy fused with log-softmax).  Reading: the loss is
# the mean over the N rows, so dz = (softmax(z) - onehot(y)) / N; no clamp.
# --------------------------------------------------------------------------

def softmax_rows(z):
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def softmax_bwd(p, dp):
    """Gradient through a row softmax p = softmax(z): dz_i = sum_j dp_j dp_j/dz_i
    with dp_j/dz_i = p_j (delta_ij - p_i), i.e. dz = p * (dp - rowsum(dp * p)).
    The tinytorch page (section 3 item 3) lists a Softmax node with its own
    backward; this is that rule written out from the derivative."""
    p = np.asarray(p, np.float64)
    dp = np.asarray(dp, np.float64)
    return p * (dp - (dp * p).sum(axis=-1, keepdims=True))


def logsumexp_rows(z):
    z = np.asarray(z, np.float64)
    m = z.max(axis=-1)
    return m + np.log(np.exp(z - m[..., None]).sum(axis=-1))


def cross_entropy_fwdbwd(z, targets, grad_scale=None):
    """Mean cross-entropy of rows of logits z [N,V] against int targets [N].

    Returns (loss, dz) with loss = mean_n(logsumexp(z_n) - z_n[y_n]) and
    dz = (softmax(z) - onehot(y)) * grad_scale, grad_scale defaulting to 1/N.
    """
    z = np.asarray(z, np.float64)
    y = np.asarray(targets, np.int64)
    n = z.shape[0]
    if grad_scale is None:
        grad_scale = 1.0 / n
    lse = logsumexp_rows(z)
    rows = np.arange(n)
    loss = float(np.mean(lse - z[rows, y]))
    dz = softmax_rows(z)
    dz[rows, y] -= 1.0
    dz *= grad_scale
    return loss, dz


def lmhead_ce_fwdbwd(h, wte, targets, store_logits=_ident, store_dlogits=_ident,
                     grad_scale=None):
    """Tied LM head followed by mean cross-entropy, forward and backward.

    z = h @ wteᵀ (tinytorch page section 3 item 6, lm_head on the final
    LayerNorm output; the head shares the token-embedding matrix, which the
    page's parameter count implies).  Returns (loss, dh, dwte, z).
    """
    h = np.asarray(h, np.float64)
    wte = np.asarray(wte, np.float64)
    z = store_logits(np.matmul(h, wte.T))
    loss, dz = cross_entropy_fwdbwd(z, targets, grad_scale)
    dz = store_dlogits(dz)
    dh = np.matmul(dz, wte)
    dwte = np.matmul(dz.T, h)
    return loss, dh, dwte, z


def argmax_rows(z):
    """Index of the row maximum, lowest index on ties (greedy decoding); a row
    holding NaN gives its first NaN (NumPy's rule: NaN ranks above every
    number)."""
    return np.argmax(np.asarray(z), axis=-1).astype(np.int64)


# --------------------------------------------------------------------------
# Causal multi-head self-attention — tinytorch page section 4 (causal mask:
# a position only sees earlier tokens; stable softmax); Forge page "最硬的一关"
# (scores divided by sqrt(d_k), upper triangle filled with -inf).
# Layout reading: qkv [B,T,3C] holds q | k | v column blocks, head h owns
# columns h*hs .. h*hs+hs-1 of each block.  No dropout.
# --------------------------------------------------------------------------

def _split_heads(qkv, n_head):
    qkv = np.asarray(qkv, np.float64)
    B, T, C3 = qkv.shape
    C = C3 // 3
    hs = C // n_head
    q = qkv[:, :, 0:C].reshape(B, T, n_head, hs).transpose(0, 2, 1, 3)
    k = qkv[:, :, C:2 * C].reshape(B, T, n_head, hs).transpose(0, 2, 1, 3)
    v = qkv[:, :, 2 * C:3 * C].reshape(B, T, n_head, hs).transpose(0, 2, 1, 3)
    return q, k, v


def _causal_probs(q, k):
    hs = q.shape[-1]
    T = q.shape[-2]
    s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(hs)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)  # j > i
    s = np.where(mask, -np.inf, s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


def attention_fwd(qkv, n_head):
    """Returns (out [B,T,C], lse [B,NH,T]) — lse is the log of each row's softmax sum."""
    q, k, v = _split_heads(qkv, n_head)
    p, lse = _causal_probs(q, k)
    o = np.matmul(p, v)  # [B,NH,T,hs]
    B, NH, T, hs = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, T, NH * hs), lse


def attention_bwd(qkv, dout, n_head):
    """Gradient of attention_fwd with respect to qkv.

    Per head, with P the causal softmax of S = q kᵀ / sqrt(hs):
      dv = Pᵀ dO ; dP = dO vᵀ ; dS = P ∘ (dP - rowsum(dP ∘ P)) ;
      dq = dS k / sqrt(hs) ; dk = dSᵀ q / sqrt(hs).
    """
    q, k, v = _split_heads(qkv, n_head)
    B, NH, T, hs = q.shape
    dO = np.asarray(dout, np.float64).reshape(B, T, NH, hs).transpose(0, 2, 1, 3)
    p, _ = _causal_probs(q, k)
    dv = np.matmul(np.swapaxes(p, -1, -2), dO)
    dp = np.matmul(dO, np.swapaxes(v, -1, -2))
    ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
    scale = 1.0 / math.sqrt(hs)
    dq = np.matmul(ds, k) * scale
    dk = np.matmul(np.swapaxes(ds, -1, -2), q) * scale
    C = NH * hs

    def merge(t):
        return t.transpose(0, 2, 1, 3).reshape(B, T, C)

    return np.concatenate([merge(dq), merge(dk), merge(dv)], axis=-1)


# --------------------------------------------------------------------------
# Embeddings — tinytorch page section 3 item 6: token embedding plus position
# embedding.  Reading: the position table is indexed by the position t.
# --------------------------------------------------------------------------

def embed_fwd(tokens, wte, wpe):
    """x0[b,t] = wte[tok[b,t]] + wpe[t].  tokens [B,T] -> [B,T,C]."""
    tok = np.asarray(tokens, np.int64)
    T = tok.shape[1]
    return np.asarray(wte, np.float64)[tok] + np.asarray(wpe, np.float64)[None, :T]


def embed_bwd(tokens, dx0, V, T_max):
    """Scatter-add of dx0 into the rows of the token table; sum over batch into wpe."""
    tok = np.asarray(tokens, np.int64)
    dx0 = np.asarray(dx0, np.float64)
    B, T, C = dx0.shape
    dwte = np.zeros((V, C))
    np.add.at(dwte, tok.reshape(-1), dx0.reshape(-1, C))
    dwpe = np.zeros((T_max, C))
    dwpe[:T] = dx0.sum(axis=0)
    return dwte, dwpe


# --------------------------------------------------------------------------
# Optimisers.
# AdamW — tinytorch page section 3 item 7 (moments m, v; bias correction with
# t = step + 1) and Forge page "核心组件清单" (AdamW: weight decay decoupled
# from the gradient update).  Reading: eps = 1e-8 added to sqrt(v_hat);
# w_new = w - lr * (m_hat / (sqrt(v_hat) + eps) + wd * w).
# SGD — tinytorch page section 8 step 5: w -= lr * g.
# --------------------------------------------------------------------------

def adamw_update(w, g, m, v, lr, beta1, beta2, eps, wd, t):
    """One AdamW step; t is 1-based.  Returns (w_new, m_new, v_new)."""
    w = np.asarray(w, np.float64)
    g = np.asarray(g, np.float64)
    m_new = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v_new = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    m_hat = m_new / (1.0 - beta1 ** t)
    v_hat = v_new / (1.0 - beta2 ** t)
    w_new = w - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * w)
    return w_new, m_new, v_new


def clip_grad_norm(grads, max_norm, eps=1e-6):
    """Global-norm gradient clipping.  The C++/CUDA page (section 3.2) keeps
    gradients in their own storage so that they can be clipped by their norm
    before the update; it prints no formula.  Reading (PyTorch's
    clip_grad_norm_): the L2 norm over every gradient entry of every tensor,
    coefficient max_norm / (norm + eps), applied only when it is below 1.
    Returns (clipped grads as float64, the norm before clipping)."""
    g64 = {k: np.asarray(v, np.float64) for k, v in grads.items()}
    total = math.sqrt(sum(float(np.sum(v * v)) for v in g64.values()))
    coef = max_norm / (total + eps)
    if coef < 1.0:
        g64 = {k: v * coef for k, v in g64.items()}
    return g64, total


def sgd_update(w, g, lr):
    return np.asarray(w, np.float64) - lr * np.asarray(g, np.float64)
