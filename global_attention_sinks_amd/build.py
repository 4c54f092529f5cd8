"""Build libmimo_attn.so (gfx950) in-tree with hipcc, and libmimo_peaks.so,
the on-box peak loops the benchmark measures beside it.

Each source compiles to its own object in parallel, then one shared library
per target links them.  Warnings are errors.  Packed FP32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmimo_attn.so")
PEAKS_LIB = os.path.join(PKG, "libmimo_peaks.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["rope.hip", "prefill.hip", "decode.hip", "backward.hip", "api.cpp"]
PEAKS_SOURCES = ["peaks.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs.  In kernels past 256 registers (dK/dV, multi-query
    # decode) the default form left the allocator copying accumulators between
    # AGPRs and VGPRs around every MFMA (383 copies per dK/dV step); with this
    # form AGPRs only hold values that wait.  Kernels under 256 are unchanged.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(extra_flags=(), out: str = LIB, verbose: bool = False) -> str:
    """Build the attention library (returned) and the peak-loop library."""
    lib = _build_one(SOURCES, out, extra_flags, verbose)
    _build_one(PEAKS_SOURCES, PEAKS_LIB, extra_flags, verbose)
    return lib


def _build_one(sources, out, extra_flags, verbose):
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            sys.stderr.write(r.stderr)
        return obj

    with ThreadPoolExecutor(len(sources)) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
