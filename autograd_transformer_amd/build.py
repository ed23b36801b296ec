"""Build libtt.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m autograd_transformer_amd.build [--jobs N] [--sanitize]
Every .hip file under csrc/ is compiled to an object in _build/ and linked
into autograd_transformer_amd/libtt.so.  Always recompiles (this is the
"does it build" step); objects are reused only within one invocation.

--sanitize builds _build/asan/libtt_asan.so instead: the same sources with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
device code is compiled as usual), for the CPU-side ABI tests
(tests/test_abi_sanitized.py runs them against it under the ASan runtime).
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


# host-only sanitizers: each -fsanitize goes to the host compilation alone
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libtt_asan.so")


def _compile(src, obj, extra=()):
    cmd = ([hipcc()] + CFLAGS + FILE_FLAGS.get(os.path.basename(src), []) + list(extra) +
           ["-c", src, "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    return err


def build(jobs=None, verbose=False, sanitize=False):
    out_dir = ASAN_DIR if sanitize else BUILD
    lib = ASAN_LIB if sanitize else LIB
    extra = SANITIZE if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(out_dir, f[:-4] + ".o") for f in srcs]
    jobs = jobs or min(8, len(srcs), os.cpu_count() or 4)
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = {ex.submit(_compile, os.path.join(CSRC, s), o, extra): s for s, o in zip(srcs, objs)}
        for f in cf.as_completed(futs):
            msg = f.result()
            if verbose and msg:
                print(futs[f], msg, file=sys.stderr)
    tmp = lib + ".tmp"
    vscript = os.path.join(out_dir, "exports.map")
    with open(vscript, "w") as f:
        f.write("{ global: tt_*; local: *; };\n")  # only the C ABI is exported
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           "-Wl,--version-script=" + vscript, "-o", tmp] + objs
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    ap.add_argument("--sanitize", action="store_true",
                    help="host AddressSanitizer + UBSan build into _build/asan/libtt_asan.so")
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, a.sanitize))
