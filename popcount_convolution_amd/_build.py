"""Build libbconv.so (hand-written HIP kernels for gfx950) in-tree with hipcc.

Each source compiles to an object under ``_build/`` in parallel; the objects
link into ``popcount_convolution_amd/libbconv.so``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbconv.so")
# longest compiles first, so they start before the pool fills
SOURCES = ("xconv_k3.hip", "xconv_k24.hip", "xconv_k5.hip", "xconv_k1.hip", "bwmma.hip", "i8mma.hip", "gemm.hip", "gemm_f4.hip",
           "xconv.hip", "xconv_small.hip", "bwconv.hip", "bconv.hip", "pack.hip", "prepack.hip", "calib.hip")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep fp32 subnormals: a negative subnormal x' must binarise to -1
    "-fno-gpu-flush-denormals-to-zero",
    # no packed fp32 VALU forms in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in SGPRs (kernels whose
    # first argument is a struct are unaffected)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbconv.so")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    """Compile every HIP source and link libbconv.so; returns its path.

    The previous library is removed first, so a failed build leaves none
    behind (callers then fail loudly instead of loading stale kernels)."""
    if os.path.exists(LIB):
        os.remove(LIB)
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
