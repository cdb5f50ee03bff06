"""Build libgemm_a8w8.so (gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libgemm_a8w8.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("a8w8_api.hip", "a8w8_kernels.hip", "a8w8_quant.hip", "a8w8_prepack.hip")]
# The benchmark's measured ceilings (streaming read, sustained fp8 MFMA): measurement aids,
# a library of their own.
CEILINGS_LIB = os.path.join(HERE, "libceilings.so")
CEILINGS_SRC = [os.path.join(HERE, "csrc", f) for f in ("read_ceiling.hip", "mfma_ceiling.hip", "cu_capacity.hip")]
# Diagnostics: the same library with the row-range kernel's per-wave timeline stamps
# compiled in (timeline.py loads it); never loaded by the product path.
TIMELINE_LIB = os.path.join(HERE, "libgemm_a8w8_timeline.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-parallel-jobs=4",
    "-Wall", "-Wno-unused-result",
    # no packed-fp32 VALU instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results go straight to VGPRs (no accvgpr copies before the scale FMA)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libgemm_a8w8.so)")


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile the HIP sources into LIB_PATH; returns the path."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB_PATH)
    build_ceilings(verbose)
    return LIB_PATH


def build_ceilings(verbose: bool = False) -> str:
    """Compile the benchmark's read- and MFMA-ceiling kernels into CEILINGS_LIB."""
    tmp = CEILINGS_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *CEILINGS_SRC]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, CEILINGS_LIB)
    return CEILINGS_LIB


def build_timeline(verbose: bool = False) -> str:
    """Compile the timeline build (-DA8W8_TIMELINE) into TIMELINE_LIB."""
    tmp = TIMELINE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, "-DA8W8_TIMELINE", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(HERE, "csrc"), "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, TIMELINE_LIB)
    return TIMELINE_LIB


if __name__ == "__main__":
    import sys
    print(build_timeline(verbose=True) if "--timeline" in sys.argv[1:] else build(verbose=True))
