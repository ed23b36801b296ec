"""The measurement probes (bench.py --probe): each runs, returns a figure in
the range the hardware allows, and rejects bad arguments.  Bounds are loose
on purpose (a probe is measurement, not parity): what they catch is a probe
that measures nothing (a loop the compiler removed, a unit mix-up) or
reports more than the part can do."""

import pytest
import torch

import autograd_transformer_amd as tt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    c = tt.Context(arena_bytes=1 << 26)
    yield c
    c.close()


def test_mfma_and_hbm_probes_are_below_the_vendor_peaks(ctx):
    mfma = tt.tt_probe_mfma(ctx, 2, 16, 2000)
    assert 500.0 < mfma < 2500.0          # TFLOP/s, dense bf16
    buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    read = tt.tt_probe_hbm(ctx, buf, copy=False)
    copy = tt.tt_probe_hbm(ctx, buf, copy=True)
    assert 1000.0 < read < 8000.0 and 1000.0 < copy < 8000.0       # GB/s


def test_lds_probes(ctx):
    alone, t0 = tt.tt_probe_lds(ctx, mfma=False)
    fed, t1 = tt.tt_probe_lds(ctx, mfma=True)
    assert t0 == 0.0
    assert 32.0 < alone <= 512.0            # bytes per clock per CU (64 banks x 4 B = 256)
    assert 8.0 < fed < alone
    assert 200.0 < t1 < 2500.0              # the MFMAs those reads feed, TFLOP/s
    buf = torch.ones(1 << 26, dtype=torch.float32, device="cuda")   # 256 MiB
    l2 = tt.tt_probe_lds_load(ctx, buf, resident=True)
    hbm = tt.tt_probe_lds_load(ctx, buf, resident=False)
    assert 1.0 < hbm < l2 <= 256.0


def test_issue_probes(ctx):
    res = [tt.tt_probe_issue(ctx, i) for i in range(len(tt.ISSUE_PROBES))]
    for (first, second), name in zip(res, tt.ISSUE_PROBES):
        assert first >= 1.0, name                  # at most one instruction per clock
        if name.endswith("1wave"):
            assert second == 0.0, name             # the second wave idles
        else:
            assert second >= 1.0, name
    # one MFMA 16x16x32 bf16 occupies its pipe for at least 8 clocks
    assert 8.0 <= res[tt.ISSUE_PROBES.index("mfma_1wave")][0] < 64.0


def test_probe_arguments_are_checked(ctx):
    with pytest.raises(tt.TTError):
        tt.tt_probe_issue(ctx, 8)
    small = torch.ones(1 << 20, dtype=torch.float32, device="cuda")  # 4 MiB: below the 64 MiB minimum
    with pytest.raises(tt.TTError):
        tt.tt_probe_lds_load(ctx, small)
    with pytest.raises(tt.TTError):
        tt.tt_probe_mfma(ctx, 9, 16, 100)
