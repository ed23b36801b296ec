"""Write sampled expected values of one full-size GPT-2 124M training step.

Calls only the CPU oracle (and the seeded input generator).  Workload: the
124M model (12 layers, C=768, 12 heads, vocab 50257, context 1024) with
synthetic weights (seed 3, N(0, 0.02), biases 0, LayerNorm 1/0), one
1024-token sequence (seed 3), bf16 mode, AdamW lr 3e-4, betas (0.9, 0.95),
eps 1e-8, weight decay 0.1, t = 1.  For every parameter tensor it stores the
gradient's L2 norm, 64 sampled gradient entries and the same entries of the
post-AdamW weights.  Run from the repository root:

    python tests/golden/make_gpt2_124m_step.py
"""

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import gpt2 as og  # noqa: E402
from autograd_transformer_amd import synthetic as syn  # noqa: E402

OUT = os.path.join(HERE, "gpt2_124m_step_b1_t1024_bf16.json")
SAMPLES = 64


def write(cfg, shape, out, producer, about=None):
    """One bf16 training step of `cfg` (weights seed 3, one 1024-token
    sequence, seed 3) through the oracle; sampled values written to `out`."""
    t0 = time.time()
    p = {k: v.astype(np.float64) for k, v in syn.gpt2_params(shape, seed=3).items()}
    tok, tgt = syn.gpt2_tokens(1, cfg.block_size, seed=3)
    zeros = {k: np.zeros_like(v) for k, v in p.items()}
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1)
    loss, grads, new_p, _, _ = og.train_step(p, zeros, dict(zeros), 1, tok, tgt, cfg, "bf16", **hp)
    rng = np.random.default_rng(2024)
    tensors = {}
    for name, _ in og.param_shapes(cfg):
        g = grads[name].reshape(-1)
        idx = np.sort(rng.choice(g.size, size=min(SAMPLES, g.size), replace=False))
        tensors[name] = dict(
            grad_norm=float(np.linalg.norm(g)),
            idx=[int(i) for i in idx],
            grad=[float(v) for v in g[idx]],
            w_new=[float(v) for v in new_p[name].reshape(-1)[idx]],
        )
    doc = dict(
        about=about or __doc__.strip().splitlines()[0],
        produced_by=f"{producer} (CPU oracle, float64)",
        workload=dict(n_layer=cfg.n_layer, n_embd=cfg.n_embd, n_head=cfg.n_head,
                      vocab=cfg.vocab, block_size=cfg.block_size,
                      B=1, T=cfg.block_size, param_seed=3, token_seed=3, mode="bf16", t=1, **hp),
        loss=float(loss),
        tensors=tensors,
        oracle_seconds=round(time.time() - t0, 1),
    )
    with open(out, "w") as f:
        json.dump(doc, f, indent=0)
    print(f"wrote {out}: loss {loss:.6f} in {time.time() - t0:.0f}s")


def main():
    write(og.GPTConfig(), syn.GPT2_124M, OUT, "tests/golden/make_gpt2_124m_step.py")


if __name__ == "__main__":
    main()
