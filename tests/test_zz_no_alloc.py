"""tt_layernorm_bwd_noalloc: the LayerNorm backward with its workspace in a
fixed device array (for callers that cannot allocate) gives what
tt_layernorm_bwd gives, on two calls in a row -- the second with fewer rows,
so it runs on workspace the first call left behind -- and refuses sizes
beyond the array.  (Named to be collected last: it must pass after every
other GPU test as well as alone.)"""

import ctypes

import numpy as np
import pytest

import oracle
import autograd_transformer_amd as tt
from autograd_transformer_amd import synthetic as syn
from tests.conftest import rel_l2
from tests.gpu_util import dev, host, zeros, tol, sync

pytestmark = pytest.mark.gpu


def _noalloc(ctx, mode, N, C, x, mean, rstd, g, dy, dx, dg, db):
    """The C entry point itself (status returned, not raised)."""
    return tt.lib().tt_layernorm_bwd_noalloc(
        ctx.handle, {"f32": 0, "bf16": 1, "fp16": 2}[mode], N, C,
        *(ctypes.c_void_p(t.data_ptr()) for t in (x, mean, rstd, g, dy, dx, dg, db)))


def _case(seed, N, C):
    x = syn.normal(seed, (N, C))
    gam = 1.0 + syn.normal(seed + 1, (C,), 0.2)
    dy = syn.normal(seed + 2, (N, C))
    res = syn.normal(seed + 3, (N, C))        # what dx holds before (+=)
    return x, gam, dy, res


@pytest.mark.parametrize("mode", ["f32", "bf16"])
def test_noalloc_matches_layernorm_bwd_twice(mode):
    ctx = tt.Context(arena_bytes=1 << 30)
    # 8192 rows use 512 workgroups (four rows per wave), then 4099 rows use
    # 513 (two per wave): the second call's workspace is larger than the
    # first's and starts with what the first left there.
    for seed, N, C in ((61, 8192, 768), (71, 4099, 768)):
        x, gam, dy, res = _case(seed, N, C)
        xd, gd, dyd = dev(x), dev(gam), dev(dy)
        beta = dev(np.zeros(C, np.float32))
        y = zeros((N, C), "bf16" if mode == "bf16" else "f32")
        mean, rstd = zeros((N,)), zeros((N,))
        tt.tt_layernorm_fwd(ctx, mode, N, C, 1e-5, xd, gd, beta, y, mean, rstd)
        out = {}
        for which in ("ref", "noalloc"):
            dx, dg, db = dev(res), zeros((C,)), zeros((C,))
            if which == "ref":
                tt.tt_layernorm_bwd(ctx, mode, N, C, xd, mean, rstd, gd, dyd, dx, dg, db)
            else:
                ctx.check(_noalloc(ctx, mode, N, C, xd, mean, rstd, gd, dyd, dx, dg, db))
            sync()
            out[which] = (host(dx), host(dg), host(db))
        for a, b in zip(out["noalloc"], out["ref"]):
            assert rel_l2(a, b) <= tol(mode), (N, rel_l2(a, b))
        # and both against the oracle's LayerNorm backward
        x64 = x.astype(np.float64)
        _, mu, rs = oracle.layernorm_fwd(x64, gam.astype(np.float64), np.zeros(C), 1e-5)
        dx_ref, dg_ref, db_ref = oracle.layernorm_bwd(x64, mu, rs, gam.astype(np.float64),
                                                      dy.astype(np.float64))
        got_dx, got_dg, got_db = out["noalloc"]
        # (the LayerNorm backward reads and writes float32 in every mode)
        assert rel_l2(got_dx - res, dx_ref) <= 1e-5
        assert rel_l2(got_dg, dg_ref) <= 1e-5
        assert rel_l2(got_db, db_ref) <= 1e-5
    ctx.close()


def test_noalloc_refuses_beyond_its_workspace():
    ctx = tt.Context(arena_bytes=1 << 28)
    C = 4096
    N = 40000          # far more partial sums than the fixed workspace holds
    t = zeros((16,))
    rc = _noalloc(ctx, "f32", N, C, t, t, t, t, t, t, t, t)
    assert rc == -1
    assert b"workspace" in tt.lib().tt_ctx_last_error(ctx.handle)
    ctx.close()
