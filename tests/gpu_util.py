"""Helpers for the GPU parity tests (imported only by tests marked ``gpu``)."""

import numpy as np

import oracle


def torch_mod():
    import torch
    return torch


def dev(a, dtype="f32"):
    """numpy -> contiguous GPU tensor (float32, bf16 or int32)."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if dtype == "i32":
        return torch.from_numpy(a.astype(np.int32)).cuda()
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
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[dtype]
    return torch.empty(shape, dtype=dt, device="cuda")


def zeros(shape, dtype="f32"):
    torch = torch_mod()
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[dtype]
    return torch.zeros(shape, dtype=dt, device="cuda")


def lowp(mode):
    return "bf16" if mode == "bf16" else "f32"


def store(mode):
    """Storage rounding the oracle applies in a mode."""
    return oracle.round_bf16 if mode == "bf16" else (lambda a: a)


def tol(mode):
    """The parity bar: rel-L2 <= 1e-5 in fp32 mode, <= 2e-2 in bf16 mode."""
    return 1e-5 if mode == "f32" else 2e-2


def sync():
    torch_mod().cuda.synchronize()
