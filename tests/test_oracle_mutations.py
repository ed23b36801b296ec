"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/`` to a temporary directory, plants one mistake by a
textual substitution (a dropped term, a wrong sign, constant, index or scale),
and runs the pin and gradient-check suites against the copy in a subprocess.
The case passes when that run FAILS.  Everything runs on the CPU.
"""

import os
import shutil
import subprocess
import sys

import pytest

from tests.conftest import ROOT

MUTANTS = {
    "gelu_constant": ("ops.py", "_GELU_A = 0.044715", "_GELU_A = 0.04715"),
    "gelu_page_backward": ("ops.py",
                           "return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du",
                           "return 0.5 * (1.0 + t) + x * np.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)"),
    "attn_scale": ("ops.py", "s = np.matmul(q, np.swapaxes(k, -1, -2)) / math.sqrt(hs)",
                   "s = np.matmul(q, np.swapaxes(k, -1, -2)) / hs"),
    "attn_mask_off_by_one": ("ops.py", "mask = np.triu(np.ones((T, T), dtype=bool), k=1)",
                             "mask = np.triu(np.ones((T, T), dtype=bool), k=2)"),
    "attn_bwd_dk_unscaled": ("ops.py", "dk = np.matmul(np.swapaxes(ds, -1, -2), q) * scale",
                             "dk = np.matmul(np.swapaxes(ds, -1, -2), q)"),
    "attn_bwd_dropped_rowsum": ("ops.py", "ds = p * (dp - (dp * p).sum(axis=-1, keepdims=True))",
                                "ds = p * dp"),
    "ln_eps_outside_sqrt": ("ops.py", "rstd = 1.0 / np.sqrt(var + eps)",
                            "rstd = 1.0 / (np.sqrt(var) + eps)"),
    "ln_unbiased_var": ("ops.py", "var = (xc * xc).mean(axis=-1)",
                        "var = (xc * xc).sum(axis=-1) / (x.shape[-1] - 1)"),
    "ln_bwd_dropped_term": ("ops.py", "dx = rstd[..., None] * (g - mg - xhat * mgx)",
                            "dx = rstd[..., None] * (g - mg)"),
    "softmax_bwd_dropped_rowsum": ("ops.py",
                                   "return p * (dp - (dp * p).sum(axis=-1, keepdims=True))",
                                   "return p * dp"),
    "loss_scale_not_undone": ("gpt2.py", "grads = {k: g / loss_scale for k, g in grads.items()}",
                              "grads = {k: g for k, g in grads.items()}"),
    "loss_scale_grows_every_step": ("gpt2.py", "if good_steps >= interval:",
                                    "if good_steps >= 1:"),
    "fp16_stored_as_bf16": ("gpt2.py", """    if mode == "fp16":
        return round_fp16""", """    if mode == "fp16":
        return round_bf16"""),
    "fp16_double_rounding": ("bf16.py", "return a.astype(np.float16).astype(np.float64)",
                             "return a.astype(np.float32).astype(np.float16).astype(np.float64)"),
    "ce_no_mean": ("ops.py", "grad_scale = 1.0 / n", "grad_scale = 1.0"),
    "adamw_no_bias_correction": ("ops.py", "v_hat = v_new / (1.0 - beta2 ** t)", "v_hat = v_new"),
    "adamw_decay_without_lr": ("ops.py",
                               "w_new = w - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * w)",
                               "w_new = w - lr * m_hat / (np.sqrt(v_hat) + eps) - wd * w"),
    "linear_bwd_wrong_sign": ("ops.py", "dx = np.matmul(dy, W.T)", "dx = -np.matmul(dy, W.T)"),
    "embed_pos_by_token": ("ops.py",
                           "return np.asarray(wte, np.float64)[tok] + np.asarray(wpe, np.float64)[None, :T]",
                           "return np.asarray(wte, np.float64)[tok] + np.asarray(wpe, np.float64)[tok % np.asarray(wpe).shape[0]]"),
    "block_missing_residual": ("gpt2.py",
                               "x1 = x + linear_fwd(att.reshape(-1, C), Wp, w[\"b_proj\"]).reshape(B, T, C)",
                               "x1 = linear_fwd(att.reshape(-1, C), Wp, w[\"b_proj\"]).reshape(B, T, C)"),
    "gelu_on_rounded_preact_swapped": ("gpt2.py", "dh = S(dg * gelu_grad(c[\"h\"]))",
                                       "dh = S(dg * gelu_grad(c[\"g\"]))"),
    "bf16_round_toward_zero": ("bf16.py", "u = u + np.uint64((1 << 44) - 1) + lsb", "u = u"),
    "argmax_highest_index_on_ties": ("ops.py",
                                     "return np.argmax(np.asarray(z), axis=-1).astype(np.int64)",
                                     "return (np.asarray(z).shape[-1] - 1 - np.argmax(np.asarray(z)[..., ::-1], axis=-1)).astype(np.int64)"),
    "clip_norm_without_sqrt": ("ops.py",
                               "total = math.sqrt(sum(float(np.sum(v * v)) for v in g64.values()))",
                               "total = sum(float(np.sum(v * v)) for v in g64.values())"),
    "greedy_takes_first_position": ("gpt2.py",
                                    "z = model_logits(params, seq, cfg, mode)[:, -1, :]",
                                    "z = model_logits(params, seq, cfg, mode)[:, 0, :]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    fname, old, new = MUTANTS[name]
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("__pycache__"))
    path = dst / fname
    src = path.read_text()
    assert src.count(old) == 1, f"mutation anchor not found once in {fname}: {old!r}"
    path.write_text(src.replace(old, new))
    env = dict(os.environ, TT_ORACLE_MUTANT_DIR=str(tmp_path), PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         "tests/test_oracle_pins.py", "tests/test_oracle_gradcheck.py"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name!r} was not caught:\n{r.stdout[-2000:]}"
