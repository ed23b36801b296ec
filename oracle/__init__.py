"""CPU oracle for the GPT-2 training step — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct NumPy float64 implementation of
what the training step computes.  It exists to check the HIP library against.
Only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import it; the product path (``autograd_transformer_amd``)
never does, and the oracle never imports the product.

Sources (page titles abbreviated; the full titles and addresses are listed in
the design notes at the repository root):

* tinytorch page — "不用PyTorch，一个头文件就能训练GPT-2：Arena内存池+自动微分的C++实现",
  section 3 ("代码实现原理") items 3-7 (MatMul, GELU, Softmax+CrossEntropy, GPT-2
  model, training loop) and section 4 (knowledge table: stable softmax,
  LayerNorm, residual, Adam, causal mask).
* Forge page — "17岁少年用C++从零构建深度学习框架Forge，精确复现GPT-2", sections
  "核心组件清单" (AdamW, log-softmax cross-entropy), "最硬的一关" (pitfall list:
  1/sqrt(d_k), causal mask, LayerNorm epsilon and variance) and
  "瓶颈分析是否合理" (softmax passes over the vocabulary).
* define-by-run page — "为什么我要从零写一个深度学习框架" (NumPy autograd), sections
  3.2 (gradient accumulation, MatMul grad shapes) and 4.2 (central-difference
  gradient check).
* microcrad page — section "Values 的工作原理" (the c = a*b worked example).
* C++/CUDA page — "从零手写C++深度学习框架：Tensor设计、Autograd与CUDA优化实战",
  section 3.4 (fp32 master weights with low-precision compute).

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` (closed forms, brute force, invariants, central
finite differences and an independent PyTorch fp64 autograd cross-check).
No function is "parity unpinned".
"""

from .bf16 import round_bf16, round_fp16
from .ops import (
    linear_fwd, linear_bwd,
    layernorm_fwd, layernorm_bwd,
    gelu_fwd, gelu_bwd,
    attention_fwd, attention_bwd,
    softmax_rows, softmax_bwd, cross_entropy_fwdbwd,
    lmhead_ce_fwdbwd,
    embed_fwd, embed_bwd,
    adamw_update, sgd_update,
    argmax_rows, clip_grad_norm,
)
from .gpt2 import (
    GPTConfig, param_shapes, param_count, zero_grads,
    block_fwd, block_bwd, model_fwd_bwd, train_step, mlp_step,
    loss_scale_update, train_step_scaled,
)

__all__ = [
    "round_bf16", "round_fp16",
    "linear_fwd", "linear_bwd", "layernorm_fwd", "layernorm_bwd",
    "gelu_fwd", "gelu_bwd", "attention_fwd", "attention_bwd",
    "softmax_rows", "softmax_bwd", "cross_entropy_fwdbwd", "lmhead_ce_fwdbwd",
    "embed_fwd", "embed_bwd", "adamw_update", "sgd_update", "argmax_rows", "clip_grad_norm",
    "GPTConfig", "param_shapes", "param_count", "zero_grads",
    "block_fwd", "block_bwd", "model_fwd_bwd", "train_step", "mlp_step",
    "loss_scale_update", "train_step_scaled",
]
