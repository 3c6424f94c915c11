"""Build libmt.so in-tree: HIP sources for gfx950 with hipcc, host-only C++
with g++, linked into one shared library next to this file.

Usage: python -m layer_streamed_amd.build  (always recompiles everything).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmt.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
# Per-source additions.  The attention kernels hold their MFMA accumulators
# and operands in VGPR form: with the default AGPR form the dK/dV kernel's
# allocation copied values between the two register files around every
# tile (several hundred v_accvgpr moves per loop trip); the instructions and
# their order are otherwise the same, so the results are too.
FILE_FLAGS = {
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}


def hip_flags(src: str) -> list:
    """hipcc flags of one HIP source."""
    return HIP_FLAGS + FILE_FLAGS.get(os.path.basename(src), [])


CXX_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-march=x86-64-v3", "-pthread", "-ffp-contract=off", "-fno-math-errno",
    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC] + hip_flags(src) + ["-c", src, "-o", obj]
    else:
        cmd = ["g++"] + CXX_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")), 16)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-pthread", "-o", tmp] + objs + [
        "-L" + os.path.join(ROCM, "lib"), "-lhsa-runtime64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
