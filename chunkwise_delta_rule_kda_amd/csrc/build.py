"""Build libkda.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m chunkwise_delta_rule_kda_amd.csrc.build   (or call build()).
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libkda.so")

SOURCES = ["kda_api.cpp", "kda_prepare.hip", "kda_recurrence.hip", "kda_fused.hip",
           "kda_decode.hip"]
HEADERS = ["kda_internal.h", "kda_device.h", "kda_recurrence_core.h", "kda_producer.h"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _run(cmd, what, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {what}")
    if verbose and res.stderr.strip():
        # hipcc's host pass does not know the packed-fp32 feature; drop that noise
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")


def build(verbose=False, out=LIB, extra_flags=(), jobs=None):
    """Compile every source (always recompiles, one hipcc per translation unit, in
    parallel) and link them into one shared library."""
    inc = ["-I", os.path.join(ROOT, "include"), "-I", HERE]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with tempfile.TemporaryDirectory(prefix="kda_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [([hipcc(), *FLAGS, *extra_flags, *inc, "-x", "hip", "-c",
                  os.path.join(HERE, s), "-o", o], s) for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=jobs) as pool:
            for f in [pool.submit(_run, c, s, verbose) for c, s in cmds]:
                f.result()
        tmp = out + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
             "the link", verbose)
    os.replace(tmp, out)
    return out


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_caller", "kda_c_caller.c")
C_CALLER = os.path.join(ROOT, "tests", "c_caller", "kda_c_caller")


def build_c_caller(verbose=False):
    """The C client used by the tests (plain C against include/kda.h and the HIP runtime,
    linked to the in-tree libkda.so)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           C_CALLER_SRC, "-o", C_CALLER, "-L", PKG, "-lkda", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../chunkwise_delta_rule_kda_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    _run(cmd, "the C client", verbose)
    return C_CALLER


if __name__ == "__main__":
    print(build(verbose=True))
