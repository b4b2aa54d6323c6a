"""Build libosm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage:  python -m online_softmax_06_amd.build [--verbose] [--resource-usage]

The library is written next to this file, so it travels with the source tree.
Every call compiles from scratch.
"""

import argparse
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libosm.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["osm_api.cpp", "softmax_rows.hip", "attn_fwd.hip", "attn_bwd.hip", "stream_copy.hip"]

ARCH = "gfx950"

# Packed-FP32 instructions are kept out of the generated code.  No fast-math
# or finite-math flag is used: the -inf guards of the online softmax and the
# overflow tests of the attention forward rely on IEEE semantics.  (Assuming
# no NaNs was measured to change nothing: bitwise equal results, times within
# 1% on the softmax, attention forward and backward workloads.)
HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libosm")
    return exe


def build(verbose=False, resource_usage=False, out=LIB_PATH):
    """Compile every source and link the shared library; return its path."""
    cmd = [hipcc()] + HIPCC_FLAGS + ["-shared", "-I", INCLUDE, "-I", CSRC]
    if resource_usage:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose or resource_usage:
        sys.stdout.write(res.stdout + res.stderr)
    os.replace(out + ".tmp", out)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose, resource_usage=a.resource_usage))


if __name__ == "__main__":
    main()
