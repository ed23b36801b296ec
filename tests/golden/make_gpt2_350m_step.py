"""Write sampled expected values of one full-size GPT-2 350M training step.

Calls only the CPU oracle (and the seeded input generator), through the
124M script's writer.  Workload: 24 layers, C=1024, 16 heads of 64, MLP
4096, vocab 50257, context 1024; synthetic weights (seed 3, N(0, 0.02),
biases 0, LayerNorm 1/0); one 1024-token sequence (seed 3); bf16 mode; AdamW
lr 3e-4, betas (0.9, 0.95), eps 1e-8, weight decay 0.1, t = 1.  Run from the
repository root:

    python tests/golden/make_gpt2_350m_step.py
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from make_gpt2_124m_step import write  # noqa: E402
from oracle import gpt2 as og  # noqa: E402
from autograd_transformer_amd import synthetic as syn  # noqa: E402

OUT = os.path.join(HERE, "gpt2_350m_step_b1_t1024_bf16.json")

if __name__ == "__main__":
    cfg = og.GPTConfig(n_layer=24, n_embd=1024, n_head=16)
    write(cfg, syn.GPT2_350M, OUT, "tests/golden/make_gpt2_350m_step.py",
          about=__doc__.strip().splitlines()[0])
