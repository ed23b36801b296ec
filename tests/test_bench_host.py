"""Host-side logic of bench.py (no GPU): the roofline of the dominant kernel,
the memory/compute bound split at the ridge point, the counter records read
from profiles/ (source-digest check, template instances combined) and the
table of HBM-bound kernels."""

import json
import os
import subprocess
import sys

import pytest

import bench
from autograd_transformer_amd.pmc_traffic import source_digest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _k(name, calls, ms, flops_per, bytes_per):
    return {"name": name, "calls": calls, "ms": ms, "flops": flops_per * calls,
            "bytes": bytes_per * calls}


def test_bound_split_at_the_ridge_point():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)   # FLOP per byte
    assert bench.bound_of(_k("a", 1, 1.0, ridge * 1e6, 1e6)) == "mfma"
    assert bench.bound_of(_k("a", 1, 1.0, 0.99 * ridge * 1e6, 1e6)) == "hbm"
    assert bench.bound_of(_k("a", 1, 1.0, 0.0, 1e6)) == "hbm"
    assert bench.bound_of(_k("a", 1, 1.0, 1e9, 0.0)) == "mfma"
    # a lower peak (fp32 MFMA) moves the ridge down
    fp32_ridge = bench.PEAK_FP32_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)
    k = _k("a", 1, 1.0, fp32_ridge * 1e6, 1e6)
    assert bench.bound_of(k, bench.PEAK_FP32_TFLOPS) == "mfma"
    assert bench.bound_of(k) == "hbm"


def test_roofline_takes_the_dominant_kernel_per_launch():
    steps, ms = 4, 10.0
    ks = [_k("small", 40, 2.0, 1e9, 1e6),
          _k("big", 8, 20.0, 2.5e12, 1e6),            # 2.5 TFLOP per launch, 2.5 ms each
          _k("mem", 4, 8.0, 0.0, 8e9)]
    r = bench.roofline(ks, steps, ms)
    assert r["kernel"] == "big" and r["bound"] == "mfma"
    assert r["avg_launch_us"] == pytest.approx(2500.0)
    assert r["achieved"] == pytest.approx(1000.0, rel=1e-6)   # 2.5e12 FLOP / 2.5 ms, TFLOP/s
    assert r["frac"] == pytest.approx(1000.0 / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    assert r["calls_per_step"] == 2 and r["share_of_step"] == pytest.approx(0.5)
    r2 = bench.roofline([ks[2]], steps, ms)
    assert r2["bound"] == "hbm" and r2["unit"] == "GB/s"
    assert r2["achieved"] == pytest.approx(4000.0)            # 8 GB per 2 ms launch


def _write_profiles(tmp_path, key, what, kernels, digest):
    os.makedirs(tmp_path / "profiles", exist_ok=True)
    with open(tmp_path / "profiles" / f"{key}_{what}.json", "w") as f:
        json.dump({"source_digest": digest, "kernels": kernels}, f)


def test_counter_records_match_digest_and_combine_instances(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    key = "w"
    traffic = {
        "gemm_kernel<float, 64, 64, 32, 2, 2, true, false, true>": {"launches": 3, "hbm_bytes_per_launch": 100},
        "gemm_kernel<float, 64, 64, 32, 2, 2, false, false, true>": {"launches": 1, "hbm_bytes_per_launch": 500},
        "gemm_kernel<__bf16, 128, 128, 64, 2, 2, true, true, true>": {"launches": 9, "hbm_bytes_per_launch": 7},
        "adamw_kernel<false>": {"launches": 1, "hbm_bytes_per_launch": 42},
    }
    busy = {
        "gemm_kernel<float, 64, 64, 32, 2, 2, true, false, true>": {"gui_active": 300, "mfma_busy": 0.2},
        "gemm_kernel<float, 64, 64, 32, 2, 2, false, false, true>": {"gui_active": 100, "mfma_busy": 0.6},
    }
    _write_profiles(tmp_path, key, "hbm_traffic", traffic, source_digest())
    _write_profiles(tmp_path, key, "mfma_busy", busy, source_digest())
    r = {"kernel": "gemm_kernel<f32>"}
    bench.counter_fields(r, key)
    assert r["traffic"] == 200              # (3 * 100 + 1 * 500) / 4 launches; bf16 instance excluded
    assert r["mfma_busy"] == pytest.approx(0.3)   # weighted by busy time: (300 * .2 + 100 * .6) / 400
    # a timer name without template arguments matches a single instance
    assert bench._counter_record(key, "hbm_traffic", "adamw_kernel", "hbm_bytes_per_launch") == 42
    assert bench._counter_record(key, "hbm_traffic", "missing_kernel", "hbm_bytes_per_launch") is None
    # summaries of other sources are not used
    _write_profiles(tmp_path, key, "hbm_traffic", traffic, "0" * 64)
    assert bench._counter_record(key, "hbm_traffic", "adamw_kernel", "hbm_bytes_per_launch") is None


def test_hbm_kernels_table(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    steps, ms = 2, 10.0
    ks = [_k("adamw_kernel", 2, 1.4, 0.0, 3.5e9),        # 0.7 ms per launch, 5 TB/s
          _k("tiny_kernel", 2, 0.01, 0.0, 1e6),           # under the share threshold
          _k("gemm", 2, 8.0, 1e13, 1e9)]                  # compute-bound: not listed
    _write_profiles(tmp_path, "w", "hbm_traffic",
                    {"adamw_kernel<false>": {"launches": 1, "hbm_bytes_per_launch": 4.2e9}},
                    source_digest())
    rows = bench.hbm_kernels(ks, steps, ms, "w")
    assert [r["kernel"] for r in rows] == ["adamw_kernel"]
    assert rows[0]["achieved_gbs"] == pytest.approx(5000.0)
    assert rows[0]["frac"] == pytest.approx(0.625)
    assert rows[0]["counter_gbs"] == pytest.approx(6000.0)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("name", ["gpt2-124m", "gpt2-350m"])
def test_step_products_cover_the_step_flops(name):
    """The vendor comparison's product list holds every GEMM of the step: its
    FLOPs are the step's algorithmic FLOPs (at the padded vocabulary the
    kernels run) less the two attention products per pass."""
    w = bench.WORKLOADS[name]
    prods = bench.step_products(**{k: w[k] for k in ("L", "C", "NH", "V", "V_pad", "T", "B")})
    gemm = sum(2.0 * m * n * k * c for m, n, k, c, _ in prods)
    attn = 3.0 * w["L"] * 2.0 * w["B"] * w["C"] * w["T"] * (w["T"] + 1)
    full = bench.step_flops(**dict(w, V=w["V_pad"]))
    assert gemm == pytest.approx(full - attn, rel=1e-12)
    # 12 products per layer and three for the tied LM head
    assert sum(p[3] for p in prods) == 12 * w["L"] + 3
