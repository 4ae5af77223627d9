"""Build the in-tree HIP library (libmxgemm.so) for gfx950 with hipcc.

Usage: python -m mxfp4_quantized_gemm_inline_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmxgemm.so")
BUILD_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"
# Packed FP32 ops are kept out of device code; no fast-math and no denormal flushing, so
# bf16 subnormals survive the quantizer.
HIP_FLAGS = ["-O3", "-std=c++20", f"--offload-arch={ARCH}", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc", "-Wall", "-Wno-unused-function"]
SOURCES = ["mx_kernels.hip", "mx_api.cpp", "mx_calib.hip", "mx_prepare_packed.hip", "mx_a16w4.hip",
           "mx_gemm_qo.hip", "mx_noalloc.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):  # host-only translation unit
        rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
        flags = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
                 "-I", os.path.join(rocm, "include")]
    else:
        flags = HIP_FLAGS
    cmd = [hipcc(), *flags, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libmxgemm.so in the package directory."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
