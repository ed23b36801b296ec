"""Write sampled expected values of the full-size fused LM head + cross-entropy.

Calls only the CPU oracle (and the seeded input generator).  Workload:
hidden [8192, 768] ~ N(0, 1) and W_emb [50257, 768] ~ N(0, 0.02), both
bf16-exact, targets uniform in [0, 50257) (seed 4); logits and their
gradient stored in bf16 (bf16 mode); mean cross-entropy over the 8192 rows.
Stores the loss, the L2 norms of dHidden and dW_emb and 256 sampled entries
of each.  Run from the repository root:

    python tests/golden/make_lmhead_ce_full.py
"""

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from autograd_transformer_amd import synthetic as syn  # noqa: E402

OUT = os.path.join(HERE, "lmhead_ce_n8192_c768_v50257_bf16.json")
N, C, V, SEED, SAMPLES = 8192, 768, 50257, 4, 256


def main():
    t0 = time.time()
    d = syn.lmhead_inputs(seed=SEED, N=N, C=C, V=V)
    S = oracle.round_bf16
    loss, dh, dwte, _ = oracle.lmhead_ce_fwdbwd(d["h"], d["wte"], d["targets"], S, S)
    rng = np.random.default_rng(2025)
    out = {}
    for name, a in (("dh", dh), ("dwte", dwte)):
        flat = a.reshape(-1)
        idx = np.sort(rng.choice(flat.size, size=SAMPLES, replace=False))
        out[name] = dict(norm=float(np.linalg.norm(flat)), idx=[int(i) for i in idx],
                         val=[float(v) for v in flat[idx]])
    doc = dict(
        about=__doc__.strip().splitlines()[0],
        produced_by="tests/golden/make_lmhead_ce_full.py (CPU oracle, float64)",
        workload=dict(N=N, C=C, V=V, seed=SEED, mode="bf16"),
        loss=float(loss),
        tensors=out,
        oracle_seconds=round(time.time() - t0, 1),
    )
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=0)
    print(f"wrote {OUT}: loss {loss:.6f} in {time.time() - t0:.0f}s")


if __name__ == "__main__":
    main()
