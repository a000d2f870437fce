"""Build libkda.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m chunkwise_delta_rule_kda_amd.csrc.build   (or call build()).
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkda.so")

SOURCES = ["kda_api.cpp", "kda_prepare.hip", "kda_recurrence.hip", "kda_decode.hip"]
HEADERS = ["kda_internal.h", "kda_device.h"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed-FP32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build(verbose=False, out=LIB, extra_flags=()):
    """Compile every source into one shared library (always recompiles)."""
    srcs = [os.path.join(HERE, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), "-I", HERE,
           "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkda.so")
    if verbose and res.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature; drop that noise
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
