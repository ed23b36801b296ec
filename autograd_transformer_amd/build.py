"""Build libtt.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m autograd_transformer_amd.build [--jobs N]
Every .hip file under csrc/ is compiled to an object in _build/ and linked
into autograd_transformer_amd/libtt.so.  Always recompiles (this is the
"does it build" step); objects are reused only within one invocation.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtt.so")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # packed fp32 instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# Per-file additions.  The MFMA probe keeps its accumulators in VGPRs: left
# to choose, the compiler holds them in AGPRs and copies every one between
# the two register files on each loop iteration, which the probe would then
# measure instead of the MFMA pipe.
FILE_FLAGS = {"probes.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm toolchain required)")
    return exe


def _compile(src, obj):
    cmd = [hipcc()] + CFLAGS + FILE_FLAGS.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return err


def build(jobs=None, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(BUILD, f[:-4] + ".o") for f in srcs]
    jobs = jobs or min(8, len(srcs), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = {ex.submit(_compile, os.path.join(CSRC, s), o): s for s, o in zip(srcs, objs)}
        for f in cf.as_completed(futs):
            msg = f.result()
            if verbose and msg:
                print(futs[f], msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    vscript = os.path.join(BUILD, "exports.map")
    with open(vscript, "w") as f:
        f.write("{ global: tt_*; local: *; };\n")  # only the C ABI is exported
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           "-Wl,--version-script=" + vscript, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose))
