"""Helpers for the GPU parity tests (imported only by tests marked ``gpu``)."""

import numpy as np

import oracle


def torch_mod():
    import torch
    return torch


def dev(a, dtype="f32"):
    """numpy -> contiguous GPU tensor (float32, bf16, fp16 or int32)."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32)).cuda()
    if dtype == "fp16":
        # numpy rounds float64 -> float16 once (torch would go through float32)
        return torch.from_numpy(a.astype(np.float16)).cuda().contiguous()
    t = torch.from_numpy(a.astype(np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda().contiguous()


def host(t):
    """GPU tensor -> float64 numpy (bf16 widened exactly)."""
    torch = torch_mod()
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def empty(shape, dtype="f32"):
    torch = torch_mod()
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16,
          "i32": torch.int32}[dtype]
    return torch.empty(shape, dtype=dt, device="cuda")


def zeros(shape, dtype="f32"):
    torch = torch_mod()
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16,
          "i32": torch.int32}[dtype]
    return torch.zeros(shape, dtype=dt, device="cuda")


def lowp(mode):
    return mode if mode in ("bf16", "fp16") else "f32"


def store(mode):
    """Storage rounding the oracle applies in a mode."""
    if mode == "bf16":
        return oracle.round_bf16
    if mode == "fp16":
        return oracle.round_fp16
    return lambda a: a


def tol(mode):
    """The parity bar: rel-L2 <= 1e-5 in fp32 mode, <= 2e-2 in bf16 mode,
    <= 1e-2 in fp16 mode (11 significant bits against bf16's 8)."""
    return {"f32": 1e-5, "bf16": 2e-2, "fp16": 1e-2}[mode]


def exact_in(mode, a):
    """Inputs exactly representable in the mode's storage format."""
    if mode == "bf16":
        return oracle.round_bf16(a)
    if mode == "fp16":
        return oracle.round_fp16(a)
    return a


def sync():
    torch_mod().cuda.synchronize()


def split_key_bias(name, got, ref, C):
    """The key third of a qkv bias has an exactly zero gradient: adding a
    constant to every key adds q·b_k to a whole score row, which the softmax
    ignores.  Returns (rest_got, rest_ref, key_got) so the rest is compared by
    rel-L2 and the key part by a noise bound."""
    if not name.endswith("b_qkv"):
        return got, ref, None
    import numpy as _np
    rest = _np.r_[0:C, 2 * C:3 * C]
    return got[rest], ref[rest], got[C:2 * C]


KEY_BIAS_NOISE = {"f32": 1e-3, "bf16": 5e-2, "fp16": 2e-2}


def check_post_adamw(w_gpu, w0, g_ref, w_ref, lr, wd, bar, grad_rms):
    """Post-AdamW weights after the first step (t = 1), where
    w1 = w0 (1 - lr wd) - lr g / (|g| + eps).  The comparison is on the
    update u = w1 - w0 (1 - lr wd), not on w1: w1 is dominated by w0 (lr/|w|
    is about 1 %), so a rel-L2 of w1 could not see a wrong update.  The update
    jumps by 2 lr when a gradient's sign changes, so entries whose oracle
    gradient is within the gradient tolerance of zero (|g| <= 0.1 rms) have
    no unique expected value: those are checked against AdamW's step bound
    |u| <= lr, the resolved entries by rel-L2 of u.  w1 is stored in float32,
    so u is observable only to one float32 ulp of w1 (about 1e-5 of lr at
    |w| = 0.05): each entry's difference is forgiven that ulp before the
    rel-L2.  Returns the rel-L2."""
    import numpy as _np
    w_gpu, w0, g_ref, w_ref = (_np.asarray(a, _np.float64).ravel() for a in (w_gpu, w0, g_ref, w_ref))
    resolved = _np.abs(g_ref) > 0.1 * grad_rms
    keep = w0 * (1 - lr * wd)
    u_gpu, u_ref = w_gpu - keep, w_ref - keep
    assert _np.all(_np.abs(u_gpu[~resolved]) <= lr * 1.001 + 1e-7 * _np.abs(w0[~resolved])), \
        "step bound"
    if not resolved.any():
        return 0.0
    ulp = _np.spacing(_np.abs(w_ref).astype(_np.float32)).astype(_np.float64)
    diff = _np.maximum(_np.abs(u_gpu - u_ref) - ulp, 0.0)
    d = _np.linalg.norm(diff[resolved])
    n = _np.linalg.norm(u_ref[resolved])
    err = d / n if n > 0 else d
    assert err <= bar, err
    return err
