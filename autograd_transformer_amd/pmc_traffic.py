"""HBM traffic and MFMA busy share per kernel launch from rocprofv3 counter runs.

    python -m autograd_transformer_amd.pmc_traffic \\
        --fetch DIR --write DIR --cal-fetch DIR --cal-write DIR --out FILE.json
    python -m autograd_transformer_amd.pmc_traffic --mfma DIR --cal-mfma DIR --out FILE.json

Each DIR is the output directory of one ``rocprofv3 --pmc FETCH_SIZE`` (or
``WRITE_SIZE``) run; ``--cal-*`` are the same counters over
``bench.py --calibrate-copy`` (a plain device copy of a known number of bytes),
which fixes the scale of each counter: bytes = counter * (known bytes / counter
reading of the copy).  The JSON lists, per kernel, the mean fetched and written
bytes per launch, and the SHA-256 of the library sources it was measured on
(``source_digest``), so a reader can tell when the figures are stale.
"""

import argparse
import collections
import csv
import glob
import hashlib
import json
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
COPY_BYTES = 1 << 30   # bench.py --calibrate-copy: bytes read and bytes written per launch


def source_digest():
    """SHA-256 over the library's HIP sources and public headers."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(_PKG, "csrc", "*.hip")) +
                   glob.glob(os.path.join(_PKG, "csrc", "*.h")) +
                   glob.glob(os.path.join(_ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(kernel_name):
    """rocprofv3's demangled name -> the name the library's timers use
    ('void (anonymous namespace)::k<1, 2>(int, ...)' -> 'k<1, 2>')."""
    n = kernel_name.replace("void ", "", 1) if kernel_name.startswith("void ") else kernel_name
    n = n.replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def _counter_means(directory, counter):
    """{short kernel name: (launches, mean KiB per launch)} of one pmc run."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    per = collections.defaultdict(list)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    per[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (len(v), sum(v) / len(v)) for k, v in per.items()}


def _copy_reading(directory, counter):
    """Mean KiB per launch of the largest copy kernel in a calibration run."""
    means = _counter_means(directory, counter)
    cands = {k: v for k, v in means.items() if "copy" in k.lower() or "Copy" in k}
    if not cands:
        raise ValueError(f"no copy kernel in {directory}: {sorted(means)}")
    return max(cands.values(), key=lambda v: v[1])[1]


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def _gpu_agent(directory):
    """SIMD and XCD counts of the profiled GPU (run_agent_info.csv)."""
    files = glob.glob(os.path.join(directory, "**", "*agent_info.csv"), recursive=True)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if int(r.get("Simd_Count", "0") or 0) > 0:
                    return int(r["Simd_Count"]), int(r.get("Num_Xcc", "1") or 1)
    raise FileNotFoundError(f"no GPU agent in {directory}")


def mfma_busy(directory, cal_directory=None):
    """Per kernel and launch: MFMA utilisation, the rocprofv3 'MfmaUtil'
    expression -- SQ_VALU_MFMA_BUSY_CYCLES summed over every SIMD over
    (GRBM_GUI_ACTIVE per XCD x SIMDs); GRBM_GUI_ACTIVE arrives summed over the
    XCDs, so it is divided by their count.  With cal_directory (the same
    counters over ``bench.py --probe``), the MFMA probe's own figure is
    returned as well: back-to-back MFMAs on every SIMD, the practical 100 %."""
    simds, xcds = _gpu_agent(directory)
    busy = _counter_means(directory, MFMA_COUNTERS[0])
    gui = _counter_means(directory, MFMA_COUNTERS[1])
    out = {}
    for k in sorted(set(busy) & set(gui)):
        n, b = busy[k]
        _, g = gui[k]
        if g > 0 and b > 0:
            out[k] = {"launches": n, "mfma_busy_cycles": round(b), "gui_active": round(g),
                      "mfma_busy": round(b / (g / xcds * simds), 4)}
    probe = None
    if cal_directory:
        cal, _ = mfma_busy(cal_directory)
        probe = max((v["mfma_busy"] for k, v in cal.items() if "mfma_probe" in k), default=None)
    return out, probe


def main_mfma(args):
    kernels, probe = mfma_busy(args.mfma, args.cal_mfma)
    out = {"workload": args.workload, "source_digest": source_digest(),
           "counters": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE; mfma_busy = "
                       "busy cycles summed over all SIMDs / (GRBM_GUI_ACTIVE per XCD x SIMDs), "
                       "rocprofv3's MfmaUtil",
           "mfma_probe_busy": probe, "kernels": kernels}
    with open(args.out, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(f"wrote {args.out}: {len(kernels)} kernels, MFMA probe {probe}")


def main():
    ap = argparse.ArgumentParser()
    for a in ("fetch", "write", "cal_fetch", "cal_write", "mfma", "cal_mfma"):
        ap.add_argument("--" + a.replace("_", "-"))
    ap.add_argument("--out", required=True)
    ap.add_argument("--workload", default="gpt2-124m B8 T1024 train step")
    args = ap.parse_args()
    if args.mfma:
        return main_mfma(args)
    if not (args.fetch and args.write and args.cal_fetch and args.cal_write):
        ap.error("--fetch, --write, --cal-fetch and --cal-write are required")
    f_scale = (COPY_BYTES / 1024.0) / _copy_reading(args.cal_fetch, "FETCH_SIZE")
    w_scale = (COPY_BYTES / 1024.0) / _copy_reading(args.cal_write, "WRITE_SIZE")
    fetch = _counter_means(args.fetch, "FETCH_SIZE")
    write = _counter_means(args.write, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) | set(write)):
        nf, fk = fetch.get(k, (0, 0.0))
        nw, wk = write.get(k, (0, 0.0))
        fb = fk * 1024.0 * f_scale
        wb = wk * 1024.0 * w_scale
        kernels[k] = {"launches": max(nf, nw), "fetch_bytes_per_launch": round(fb),
                      "write_bytes_per_launch": round(wb), "hbm_bytes_per_launch": round(fb + wb)}
    out = {"workload": args.workload, "source_digest": source_digest(),
           "counters": "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by a "
                       "1 GiB device copy",
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": kernels}
    with open(args.out, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(f"wrote {args.out}: {len(kernels)} kernels, scales fetch {f_scale:.3f} write {w_scale:.3f}")


if __name__ == "__main__":
    main()
