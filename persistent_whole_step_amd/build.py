"""Build libtk.so (host scheduler + C ABI + the gfx950 persistent kernel) in-tree.

Every HIP translation unit is compiled for gfx950 only, without fused
multiply-add contraction (pointwise results must equal IEEE binary32 step by
step), without denormal flushing, and with packed-fp32 instruction selection
turned off.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtk.so")
OBJ = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = ["-std=c++17", "-O3", "-fPIC", "-Wall", "-Wno-unused-function", "-Wno-unused-result"]
# -falign-loops=64: loop heads start on a 64-byte instruction-cache line, so
# where a hot loop falls in a line no longer shifts with unrelated code
DEVICE = ["--offload-arch=gfx950", "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-munsafe-fp-atomics", "-falign-loops=64"]
HOST_SOURCES = ["tk_ir.cpp", "tk_sched.cpp"]
HIP_SOURCES = ["tk_api.cpp", "tk_device.hip"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if src in HOST_SOURCES:
        cmd = [HIPCC, "-x", "c++", *COMMON, "-ffp-contract=off", "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        lang = ["-x", "hip"]
        cmd = [HIPCC, *lang, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = HOST_SOURCES + HIP_SOURCES
    with cf.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
