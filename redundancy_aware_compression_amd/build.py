"""Builds librkv.so (the gfx950 HIP kernels and the C-ABI host layer) and
librkv_peaks.so (peak microbenchmarks, measurement only) in place.

    python -m redundancy_aware_compression_amd.build

Every .hip file is compiled with hipcc for gfx950 only; packed-FP32 VALU
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "librkv.so")
PEAKS_SRC = os.path.join(PKG, "peaks", "rkv_peaks.hip")
PEAKS_LIB_PATH = os.path.join(PKG, "librkv_peaks.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# MFMA accumulators in VGPRs (no accumulator-register copies before the epilogues)
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]


def sources():
    hip = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False) -> str:
    hip, cpp = sources()
    with tempfile.TemporaryDirectory(prefix="rkv_build_") as tmp:
        objs = []
        for src in hip + cpp:
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            flags = COMMON_FLAGS + (DEVICE_FLAGS if src.endswith(".hip") else [])
            cmd = [HIPCC] + flags + ["-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{err}")
            if err.strip() and verbose:
                print(err)
            objs.append(obj)
        tmp_so = LIB_PATH + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_so] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp_so, LIB_PATH)
    build_peaks(verbose)
    return LIB_PATH


def build_peaks(verbose: bool = False) -> str:
    """librkv_peaks.so: the peak microbenchmarks (measurement only)."""
    tmp_so = PEAKS_LIB_PATH + ".tmp"
    cmd = [HIPCC] + COMMON_FLAGS + DEVICE_FLAGS + ["-shared", PEAKS_SRC, "-o", tmp_so]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
        raise RuntimeError(f"hipcc failed on {PEAKS_SRC}:\n{err}")
    os.replace(tmp_so, PEAKS_LIB_PATH)
    return PEAKS_LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
