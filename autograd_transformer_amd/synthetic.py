"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers: it holds none of the training step's
arithmetic and imports neither the HIP library nor the CPU oracle.  Recipe:

* every workload has its own ``numpy.random.SeedSequence(seed)``; one child
  stream is spawned per tensor, in a fixed order, so adding a tensor never
  changes the values of the ones before it;
* values are drawn in float64 and cast to float32; tensors the workload
  declares as bf16 are additionally rounded to the nearest bf16 value (torch's
  float32 -> bfloat16 conversion, round to nearest even) and returned as
  float32 arrays holding bf16-exact values;
* weight matrices (including the token and position tables) ~ N(0, 0.02),
  LayerNorm gamma = 1 and beta = 0, biases 0 unless ``bias_std`` asks for a
  perturbed variant (used by tests to exercise the bias paths);
* token ids are uniform integers in [0, V); a [B, T+1] draw gives the inputs
  ([:, :T]) and the next-token targets ([:, 1:]).

The pages train on TinyShakespeare with pretrained weights; neither is used:
these draws stand in for them with the same shapes (context 1024, vocabulary
50257), not the same text statistics.
"""

from dataclasses import dataclass

import numpy as np


def _streams(seed, n):
    ss = np.random.SeedSequence(seed)
    return [np.random.default_rng(s) for s in ss.spawn(n)]


def _bf16_exact(a):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


# ----------------------------------------------------------------- tiny MLP

def mlp_inputs(seed=1, batch=64, n_in=3, hidden=32, classes=4):
    """x[64,3], W1[3,32], b1[32], W2[32,4], b2[4] ~ N(0,1); labels ~ U{0..3}."""
    r = _streams(seed, 6)
    return dict(
        x=_normal(r[0], (batch, n_in)),
        W1=_normal(r[1], (n_in, hidden)), b1=_normal(r[2], (hidden,)),
        W2=_normal(r[3], (hidden, classes)), b2=_normal(r[4], (classes,)),
        labels=r[5].integers(0, classes, size=(batch,)).astype(np.int32),
    )


# ----------------------------------------------------------- one GPT-2 block

LAYER_TENSORS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj",
                 "ln2_g", "ln2_b", "w_fc", "b_fc", "w_fcp", "b_fcp")


def _layer_weights(rngs, C, F, w_std, bias_std, ln_std):
    """Draw one block's tensors from 12 streams, in LAYER_TENSORS order."""
    shapes = dict(ln1_g=(C,), ln1_b=(C,), w_qkv=(C, 3 * C), b_qkv=(3 * C,),
                  w_proj=(C, C), b_proj=(C,), ln2_g=(C,), ln2_b=(C,),
                  w_fc=(C, F), b_fc=(F,), w_fcp=(F, C), b_fcp=(C,))
    out = {}
    for rng, name in zip(rngs, LAYER_TENSORS):
        shp = shapes[name]
        if name.startswith("w_"):
            out[name] = _normal(rng, shp, w_std)
        elif name.endswith("_g"):
            out[name] = (1.0 + _normal(rng, shp, ln_std)) if ln_std else np.ones(shp, np.float32)
        elif name.startswith("ln"):
            out[name] = _normal(rng, shp, ln_std) if ln_std else np.zeros(shp, np.float32)
        else:
            out[name] = _normal(rng, shp, bias_std) if bias_std else np.zeros(shp, np.float32)
        out[name] = out[name].astype(np.float32)
    return out


def block_inputs(seed=2, B=4, T=256, C=768, n_head=12, F=None, w_std=0.02,
                 bias_std=0.0, ln_std=0.0):
    """Single block workload: x[B,T,C] ~ N(0,1), weights ~ N(0, w_std),
    LN gamma=1 beta=0, biases 0 (or perturbed), upstream grad dy ~ N(0,1)."""
    F = 4 * C if F is None else F
    r = _streams(seed, 14)
    w = _layer_weights(r[1:13], C, F, w_std, bias_std, ln_std)
    return dict(x=_normal(r[0], (B, T, C)), w=w, dy=_normal(r[13], (B, T, C)),
                B=B, T=T, C=C, n_head=n_head, F=F)


# ------------------------------------------------------------ whole GPT-2

@dataclass(frozen=True)
class ModelShape:
    n_layer: int
    n_embd: int
    n_head: int
    vocab: int = 50257
    block_size: int = 1024


GPT2_124M = ModelShape(12, 768, 12)
GPT2_350M = ModelShape(24, 1024, 16)


def gpt2_params(shape: ModelShape, seed=3, w_std=0.02, bias_std=0.0, ln_std=0.0):
    """All trainable tensors of a GPT-2 of the given shape, as float32 arrays.

    Order of streams: wte, wpe, then 12 per layer, then lnf_g, lnf_b."""
    C, F, L = shape.n_embd, 4 * shape.n_embd, shape.n_layer
    r = _streams(seed, 2 + 12 * L + 2)
    p = {"wte": _normal(r[0], (shape.vocab, C), w_std),
         "wpe": _normal(r[1], (shape.block_size, C), w_std)}
    for l in range(L):
        lw = _layer_weights(r[2 + 12 * l: 2 + 12 * (l + 1)], C, F, w_std, bias_std, ln_std)
        for k, v in lw.items():
            p[f"h{l}.{k}"] = v
    if ln_std:
        p["lnf_g"] = (1.0 + _normal(r[-2], (C,), ln_std)).astype(np.float32)
        p["lnf_b"] = _normal(r[-1], (C,), ln_std)
    else:
        p["lnf_g"] = np.ones((C,), np.float32)
        p["lnf_b"] = np.zeros((C,), np.float32)
    return p


def gpt2_tokens(B, T, vocab=50257, seed=3):
    """Uniform token ids [B, T+1]; returns (tokens [B,T], targets [B,T]) int32."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7919]))
    ids = rng.integers(0, vocab, size=(B, T + 1)).astype(np.int32)
    return np.ascontiguousarray(ids[:, :T]), np.ascontiguousarray(ids[:, 1:])


# ------------------------------------------------------ LM head + CE alone

def lmhead_inputs(seed=4, N=8192, C=768, V=50257, h_std=1.0, w_std=0.02):
    """hidden[N,C] ~ N(0,1) and W_emb[V,C] ~ N(0,0.02), both bf16-exact;
    targets ~ U[0,V)."""
    r = _streams(seed, 3)
    return dict(
        h=_bf16_exact(_normal(r[0], (N, C), h_std)),
        wte=_bf16_exact(_normal(r[1], (V, C), w_std)),
        targets=r[2].integers(0, V, size=(N,)).astype(np.int32),
    )


def normal(seed, shape, std=1.0):
    """A single seeded N(0, std^2) float32 tensor (op-level tests)."""
    return _normal(np.random.default_rng(np.random.SeedSequence(seed)), shape, std)


def bf16_exact(a):
    """Round a float32 array to bf16-exact values (input preparation)."""
    return _bf16_exact(a)
