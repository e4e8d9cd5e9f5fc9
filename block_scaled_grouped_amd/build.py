"""Builds libbsg.so (HIP for gfx950) in-tree with hipcc.

    python -m block_scaled_grouped_amd.build [-v]

Every source compiles every time (the caller asked for a build); objects go to
``block_scaled_grouped_amd/_build/`` and the library to
``block_scaled_grouped_amd/libbsg.so``.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libbsg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

KERNEL_SOURCES = ["offsets.hip", "quantize_mxfp8.hip", "quantize_nvfp4.hip", "gemm_mxfp8.hip",
                  "gemm_nvfp4.hip"]
HOST_SOURCES = ["api.cpp"]

# Packed-fp32 VALU ops are turned off for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is noise
    lines = [ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build step failed: %s\n%s" % (" ".join(cmd), "\n".join(lines)))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose=False, jobs=None):
    """Compiles all sources and links libbsg.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 1)
    steps = []
    objs = []
    for src in KERNEL_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([HIPCC] + DEVICE_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        steps.append([HIPCC] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
