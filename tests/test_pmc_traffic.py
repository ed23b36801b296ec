"""The rocprofv3 counter post-processing (autograd_transformer_amd/pmc_traffic.py)
on small synthetic counter files: kernel-name shortening, the copy
calibration of FETCH_SIZE / WRITE_SIZE, per-launch means, and the MFMA
utilisation formula (busy cycles over all SIMDs / (GUI-active cycles per XCD
x SIMD count))."""

import csv
import json
import os
import sys

import pytest

from autograd_transformer_amd import pmc_traffic as pt

FIELDS = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size",
          "Counter_Name", "Counter_Value"]


def _counters(directory, rows):
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": kernel,
                        "Grid_Size": 256, "Workgroup_Size": 256, "Counter_Name": counter,
                        "Counter_Value": value})


def _agent(directory, simds=1024, xcc=8):
    with open(os.path.join(directory, "run_agent_info.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Node_Id", "Agent_Type", "Simd_Count", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Node_Id": 0, "Agent_Type": "CPU", "Simd_Count": 0, "Num_Xcc": 1})
        w.writerow({"Node_Id": 1, "Agent_Type": "GPU", "Simd_Count": simds, "Num_Xcc": xcc})


GEMM = "void (anonymous namespace)::gemm_kernel<256, 128, true>(tt_gemm_detail::GemmParams)"
COPY = "__amd_rocclr_copyBuffer"


def test_short_name():
    assert pt.short_name(GEMM) == "gemm_kernel<256, 128, true>"
    assert pt.short_name("void f(int)") == "f"
    assert pt.short_name("void (anonymous namespace)::k<(unsigned char)1>(int)") == \
        "k<(unsigned char)1>"
    assert pt.short_name(COPY) == COPY


def test_traffic_scaled_by_the_copy(tmp_path, monkeypatch):
    d = str(tmp_path)
    # the 1 GiB calibration copy: FETCH_SIZE reads half of it, WRITE_SIZE all of it
    _counters(f"{d}/cal_f", [(COPY, "FETCH_SIZE", 524288.0), (COPY, "FETCH_SIZE", 524288.0)])
    _counters(f"{d}/cal_w", [(COPY, "WRITE_SIZE", 1048576.0)])
    _counters(f"{d}/f", [(GEMM, "FETCH_SIZE", 1000.0), (GEMM, "FETCH_SIZE", 3000.0)])
    _counters(f"{d}/w", [(GEMM, "WRITE_SIZE", 500.0), (GEMM, "WRITE_SIZE", 500.0)])
    out = f"{d}/t.json"
    monkeypatch.setattr(sys, "argv", ["pmc_traffic", "--fetch", f"{d}/f", "--write", f"{d}/w",
                                      "--cal-fetch", f"{d}/cal_f", "--cal-write", f"{d}/cal_w",
                                      "--out", out])
    pt.main()
    rec = json.load(open(out))
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    k = rec["kernels"]["gemm_kernel<256, 128, true>"]
    assert k["launches"] == 2
    assert k["fetch_bytes_per_launch"] == 2000 * 1024 * 2     # mean KiB x 1024 x scale
    assert k["write_bytes_per_launch"] == 500 * 1024
    assert k["hbm_bytes_per_launch"] == 2000 * 2048 + 500 * 1024
    assert rec["source_digest"] == pt.source_digest()


def test_calibration_needs_a_copy_kernel(tmp_path):
    _counters(str(tmp_path), [(GEMM, "FETCH_SIZE", 1.0)])
    with pytest.raises(ValueError):
        pt._copy_reading(str(tmp_path), "FETCH_SIZE")


def test_mfma_busy_formula(tmp_path):
    d = str(tmp_path / "run")
    _counters(d, [(GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 1000.0), (GEMM, "GRBM_GUI_ACTIVE", 80.0),
                  (GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", 3000.0), (GEMM, "GRBM_GUI_ACTIVE", 80.0)])
    _agent(d, simds=1024, xcc=8)
    cal = str(tmp_path / "cal")
    probe = "void (anonymous namespace)::mfma_probe_kernel<32>(int, float*)"
    _counters(cal, [(probe, "SQ_VALU_MFMA_BUSY_CYCLES", 9216.0), (probe, "GRBM_GUI_ACTIVE", 80.0)])
    _agent(cal, simds=1024, xcc=8)
    kernels, probe_busy = pt.mfma_busy(d, cal)
    k = kernels["gemm_kernel<256, 128, true>"]
    # mean busy 2000 cycles over 1024 SIMDs against 80 / 8 = 10 GUI-active cycles per XCD
    assert k["launches"] == 2 and k["mfma_busy"] == pytest.approx(2000 / (10 * 1024), abs=1e-4)
    assert probe_busy == pytest.approx(9216 / (10 * 1024), abs=1e-4)
