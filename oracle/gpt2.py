"""GPT-2 block, model and training step in NumPy float64 (test infrastructure only).

Model structure — tinytorch page section 3 item 6 ("GPT-2模型"): token plus
position embedding, then per layer LN1 -> attention -> +x -> LN2 -> MLP -> +x
(pre-LN), then the final LayerNorm and the LM head.  Training loop — same page,
item 7: forward, zero the gradients, backward, Adam update.  Readings taken
where the page is silent or simplified:

* loss on every position with next-token targets (the page's last-position-only
  loss is marked as a simplification), mean over all B*T positions;
* the LM head is tied to the token embedding (the page's parameter count,
  124,475,904 at the padded vocabulary 50304, matches a tied head exactly);
* weight matrices are [in, out]; MLP width F = 4C; LayerNorm eps 1e-5;
* AdamW decays every parameter (no exemption list on the pages).

Precision modes.  ``mode="f32"``: no storage rounding (float64 maths
throughout).  ``mode="fp16"``: as bf16 below with IEEE binary16 storage, used
with loss scaling (``model_fwd_bwd(loss_scale=...)``, ``train_step_scaled``).  ``mode="bf16"`` (the C++/CUDA page, section 3.4: fp32 master
weights, low-precision compute): the four block weight matrices and the tied
LM-head matrix enter their products as bf16-rounded copies of the fp32 master
values, and the tensors the training step stores as bf16 (LayerNorm outputs,
qkv, attention output, MLP pre-activation and GELU output, logits and their
gradient, and every activation gradient that feeds a product) are rounded to
bf16 where they are stored.  All arithmetic stays float64.  Biases, LayerNorm
parameters, embeddings used by the gather, the residual stream and all weight
gradients stay full precision.
"""

from dataclasses import dataclass

import numpy as np

from .bf16 import round_bf16, round_fp16
from .ops import (
    linear_fwd, linear_bwd, layernorm_fwd, layernorm_bwd, gelu_fwd, gelu_grad,
    attention_fwd, attention_bwd, lmhead_ce_fwdbwd, cross_entropy_fwdbwd,
    embed_fwd, embed_bwd, adamw_update, sgd_update, argmax_rows,
)


@dataclass(frozen=True)
class GPTConfig:
    n_layer: int = 12
    n_embd: int = 768
    n_head: int = 12
    vocab: int = 50257
    block_size: int = 1024      # rows of the position table
    mlp_mult: int = 4
    ln_eps: float = 1e-5

    @property
    def F(self):
        return self.mlp_mult * self.n_embd


LAYER_PARAMS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj",
                "ln2_g", "ln2_b", "w_fc", "b_fc", "w_fcp", "b_fcp")
MATRIX_PARAMS = ("w_qkv", "w_proj", "w_fc", "w_fcp")


def param_shapes(cfg: GPTConfig, vocab_rows=None):
    """Ordered (name, shape) list of every trainable tensor."""
    V = cfg.vocab if vocab_rows is None else vocab_rows
    C, F = cfg.n_embd, cfg.F
    out = [("wte", (V, C)), ("wpe", (cfg.block_size, C))]
    for l in range(cfg.n_layer):
        out += [
            (f"h{l}.ln1_g", (C,)), (f"h{l}.ln1_b", (C,)),
            (f"h{l}.w_qkv", (C, 3 * C)), (f"h{l}.b_qkv", (3 * C,)),
            (f"h{l}.w_proj", (C, C)), (f"h{l}.b_proj", (C,)),
            (f"h{l}.ln2_g", (C,)), (f"h{l}.ln2_b", (C,)),
            (f"h{l}.w_fc", (C, F)), (f"h{l}.b_fc", (F,)),
            (f"h{l}.w_fcp", (F, C)), (f"h{l}.b_fcp", (C,)),
        ]
    out += [("lnf_g", (C,)), ("lnf_b", (C,))]
    return out


def param_count(cfg: GPTConfig, vocab_rows=None):
    return int(sum(int(np.prod(s)) for _, s in param_shapes(cfg, vocab_rows)))


def zero_grads(params):
    return {k: np.zeros_like(np.asarray(v, np.float64)) for k, v in params.items()}


def _store_fn(mode):
    if mode == "f32":
        return lambda a: a
    if mode == "bf16":
        return round_bf16
    if mode == "fp16":
        return round_fp16
    raise ValueError(f"unknown mode {mode!r}")


# --------------------------------------------------------------------------
# One transformer block (pre-LN), forward and hand-derived backward.
# --------------------------------------------------------------------------

def block_fwd(x, w, n_head, mode="f32", eps=1e-5):
    """x [B,T,C] (full precision residual stream); w: dict of block tensors
    keyed by LAYER_PARAMS.  Returns (y, cache)."""
    S = _store_fn(mode)
    x = np.asarray(x, np.float64)
    B, T, C = x.shape
    Wq, Wp, Wf, Wfp = (S(np.asarray(w[k], np.float64)) for k in MATRIX_PARAMS)

    u, mu1, rs1 = layernorm_fwd(x, w["ln1_g"], w["ln1_b"], eps)
    u = S(u)
    qkv = S(linear_fwd(u.reshape(-1, C), Wq, w["b_qkv"]).reshape(B, T, 3 * C))
    att, lse = attention_fwd(qkv, n_head)
    att = S(att)
    x1 = x + linear_fwd(att.reshape(-1, C), Wp, w["b_proj"]).reshape(B, T, C)

    v2, mu2, rs2 = layernorm_fwd(x1, w["ln2_g"], w["ln2_b"], eps)
    v2 = S(v2)
    hpre = linear_fwd(v2.reshape(-1, C), Wf, w["b_fc"])
    h = S(hpre)
    g = S(gelu_fwd(hpre))
    y = x1 + linear_fwd(g, Wfp, w["b_fcp"]).reshape(B, T, C)

    cache = dict(x=x, u=u, mu1=mu1, rs1=rs1, qkv=qkv, att=att, lse=lse, x1=x1,
                 v2=v2, mu2=mu2, rs2=rs2, h=h, g=g,
                 Wq=Wq, Wp=Wp, Wf=Wf, Wfp=Wfp)
    return y, cache


def block_bwd(cache, w, dy, n_head, mode="f32"):
    """dy [B,T,C] full precision.  Returns (dx, grads) with grads keyed by
    LAYER_PARAMS (each the gradient of this call alone)."""
    S = _store_fn(mode)
    c = cache
    x, x1 = c["x"], c["x1"]
    B, T, C = x.shape
    dy = np.asarray(dy, np.float64)
    dyb = S(dy).reshape(-1, C)
    gr = {}

    # MLP down-projection, then GELU (uses the stored pre-activation h).
    dg, gr["w_fcp"], gr["b_fcp"] = linear_bwd(c["g"], c["Wfp"], dyb)
    dh = S(dg * gelu_grad(c["h"]))
    # MLP up-projection.
    dv2, gr["w_fc"], gr["b_fc"] = linear_bwd(c["v2"].reshape(-1, C), c["Wf"], dh)
    dln2, gr["ln2_g"], gr["ln2_b"] = layernorm_bwd(
        x1, c["mu2"], c["rs2"], w["ln2_g"], dv2.reshape(B, T, C))
    dx1 = dy + dln2
    dx1b = S(dx1).reshape(-1, C)

    # Attention projection.
    datt, gr["w_proj"], gr["b_proj"] = linear_bwd(c["att"].reshape(-1, C), c["Wp"], dx1b)
    datt = S(datt)
    dqkv = S(attention_bwd(c["qkv"], datt.reshape(B, T, C), n_head))
    du, gr["w_qkv"], gr["b_qkv"] = linear_bwd(
        c["u"].reshape(-1, C), c["Wq"], dqkv.reshape(-1, 3 * C))
    dln1, gr["ln1_g"], gr["ln1_b"] = layernorm_bwd(
        x, c["mu1"], c["rs1"], w["ln1_g"], du.reshape(B, T, C))
    dx = dx1 + dln1
    return dx, gr


# --------------------------------------------------------------------------
# Whole model: embedding -> blocks -> final LayerNorm -> tied head + CE.
# --------------------------------------------------------------------------

def _layer_w(params, l):
    return {k: params[f"h{l}.{k}"] for k in LAYER_PARAMS}


def model_fwd_bwd(params, tokens, targets, cfg: GPTConfig, mode="f32", loss_scale=1.0):
    """Forward and backward of the mean next-token loss over all B*T positions.

    Sequences are processed one at a time with gradients accumulated (the
    result is the batched one: every per-position term carries the same
    1/(B*T) factor).  Returns (loss, grads) with grads keyed like params.

    loss_scale (the C++/CUDA page, section 3.4, loss scaling for FP16): the
    backward starts from loss_scale times the loss gradient, so every stored
    activation gradient carries that factor (and may overflow the storage
    format to infinity); the returned weight gradients are divided by it
    again.  Non-finite values are left to propagate; the caller checks.
    """
    if mode == "fp16":
        with np.errstate(over="ignore", invalid="ignore"):
            return _model_fwd_bwd(params, tokens, targets, cfg, mode, loss_scale)
    return _model_fwd_bwd(params, tokens, targets, cfg, mode, loss_scale)


def _model_fwd_bwd(params, tokens, targets, cfg, mode, loss_scale):
    S = _store_fn(mode)
    tokens = np.asarray(tokens, np.int64)
    targets = np.asarray(targets, np.int64)
    B, T = tokens.shape
    N = B * T
    V, C = cfg.vocab, cfg.n_embd
    grads = zero_grads(params)
    wte = np.asarray(params["wte"], np.float64)
    wte_head = S(wte[:V])
    loss = 0.0
    for b in range(B):
        tok = tokens[b:b + 1]
        x = embed_fwd(tok, wte, params["wpe"])
        caches = []
        for l in range(cfg.n_layer):
            x, cch = block_fwd(x, _layer_w(params, l), cfg.n_head, mode, cfg.ln_eps)
            caches.append(cch)
        f, muf, rsf = layernorm_fwd(x, params["lnf_g"], params["lnf_b"], cfg.ln_eps)
        f = S(f)
        lb, df, dwte_head, _ = lmhead_ce_fwdbwd(
            f.reshape(-1, C), wte_head, targets[b], store_logits=S,
            store_dlogits=S, grad_scale=loss_scale / N)
        loss += lb * T / N
        grads["wte"][:V] += dwte_head
        dx, dg, dbt = layernorm_bwd(x, muf, rsf, params["lnf_g"], df.reshape(1, T, C))
        grads["lnf_g"] += dg
        grads["lnf_b"] += dbt
        for l in reversed(range(cfg.n_layer)):
            dx, gl = block_bwd(caches[l], _layer_w(params, l), dx, cfg.n_head, mode)
            for k, gv in gl.items():
                grads[f"h{l}.{k}"] += gv
        dwte_e, dwpe = embed_bwd(tok, dx, wte.shape[0], params["wpe"].shape[0])
        grads["wte"] += dwte_e
        grads["wpe"] += dwpe
    if loss_scale != 1.0:
        grads = {k: g / loss_scale for k, g in grads.items()}
    return loss, grads


def model_logits(params, tokens, cfg: GPTConfig, mode="f32"):
    """Forward only: the tied head's logits [B, T, V] at every position, stored
    in the mode's dtype -- the forward of the training step (tinytorch page
    section 3 items 6-7) without the loss."""
    S = _store_fn(mode)
    tokens = np.asarray(tokens, np.int64)
    B, T = tokens.shape
    V = cfg.vocab
    wte = np.asarray(params["wte"], np.float64)
    wte_head = S(wte[:V])
    out = np.empty((B, T, V))
    for b in range(B):
        x = embed_fwd(tokens[b:b + 1], wte, params["wpe"])
        for l in range(cfg.n_layer):
            x, _ = block_fwd(x, _layer_w(params, l), cfg.n_head, mode, cfg.ln_eps)
        f, _, _ = layernorm_fwd(x, params["lnf_g"], params["lnf_b"], cfg.ln_eps)
        out[b] = S(np.matmul(S(f)[0], wte_head.T))
    return out


def greedy_generate(params, prompt, n_new, cfg: GPTConfig, mode="f32"):
    """Greedy generation by its definition (the Forge page's inference loop
    picks the most likely next token; the pages' missing KV cache is only a way
    to compute the same thing faster): every new token is the argmax (lowest
    index on ties) of the last position's logits of the whole sequence so far,
    recomputed from scratch.  Returns (tokens [B, T0 + n_new], the logits of
    each step [n_new, B, V])."""
    seq = np.asarray(prompt, np.int64)
    steps = []
    for _ in range(n_new):
        z = model_logits(params, seq, cfg, mode)[:, -1, :]
        steps.append(z)
        seq = np.concatenate([seq, argmax_rows(z)[:, None]], axis=1)
    return seq, np.stack(steps)


def loss_scale_update(scale, good_steps, overflow, interval=1000, growth=1.001, backoff=0.5):
    """Dynamic loss scaling (the C++/CUDA page, section 3.4): after a step whose
    gradients hold inf or NaN the scale is halved and the step is dropped;
    after `interval` consecutive clean steps it grows by the factor 1.001.
    Reading: the clean-step count restarts after every change of the scale.
    Returns (new_scale, new_good_steps)."""
    if overflow:
        return scale * backoff, 0
    good_steps += 1
    if good_steps >= interval:
        return scale * growth, 0
    return scale, good_steps


def train_step_scaled(params, m, v, t, tokens, targets, cfg: GPTConfig, scale, good_steps,
                      mode="fp16", lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1):
    """One FP16 training step with dynamic loss scaling: the backward at the
    current scale, then either AdamW on the unscaled gradients (all finite) or
    no update (any inf or NaN), and the scale update.

    Returns (loss, grads, new_params, new_m, new_v, new_scale, new_good_steps,
    skipped); a skipped step returns the inputs unchanged."""
    loss, grads = model_fwd_bwd(params, tokens, targets, cfg, mode, loss_scale=scale)
    skipped = not all(np.all(np.isfinite(g)) for g in grads.values())
    new_scale, new_good = loss_scale_update(scale, good_steps, skipped)
    if skipped:
        return loss, grads, params, m, v, new_scale, new_good, True
    new_p, new_m, new_v = {}, {}, {}
    for k in params:
        new_p[k], new_m[k], new_v[k] = adamw_update(
            params[k], grads[k], m[k], v[k], lr, beta1, beta2, eps, wd, t)
    return loss, grads, new_p, new_m, new_v, new_scale, new_good, False


def train_step(params, m, v, t, tokens, targets, cfg: GPTConfig, mode="f32",
               lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1):
    """One training step: zero grads, forward, backward, AdamW on every tensor.

    Returns (loss, grads, new_params, new_m, new_v).
    """
    loss, grads = model_fwd_bwd(params, tokens, targets, cfg, mode)
    new_p, new_m, new_v = {}, {}, {}
    for k in params:
        new_p[k], new_m[k], new_v[k] = adamw_update(
            params[k], grads[k], m[k], v[k], lr, beta1, beta2, eps, wd, t)
    return loss, grads, new_p, new_m, new_v


def mlp_step(x, W1, b1, W2, b2, labels, lr=0.1):
    """Tiny classifier: Linear -> tanh-GELU -> Linear -> softmax -> mean CE,
    full backward, one SGD step (tinytorch page, section 8 step 5 example).

    Returns (loss, grads dict, new params dict, logits)."""
    x = np.asarray(x, np.float64)
    hpre = linear_fwd(x, W1, b1)
    h = gelu_fwd(hpre)
    z = linear_fwd(h, W2, b2)
    loss, dz = cross_entropy_fwdbwd(z, labels)
    dh, dW2, db2 = linear_bwd(h, W2, dz)
    dhpre = dh * gelu_grad(hpre)
    _, dW1, db1 = linear_bwd(x, W1, dhpre)
    grads = dict(W1=dW1, b1=db1, W2=dW2, b2=db2)
    old = dict(W1=W1, b1=b1, W2=W2, b2=b2)
    new = {k: sgd_update(old[k], grads[k], lr) for k in old}
    return loss, grads, new, z
