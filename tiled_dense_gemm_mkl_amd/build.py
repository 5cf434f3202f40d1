"""Build libgemm_mkl.so (the HIP library) in-tree for gfx950.

Usage: ``python -m tiled_dense_gemm_mkl_amd.build`` (or ``build()`` from Python).
Each translation unit under csrc/ is compiled by hipcc in parallel, then the
objects are linked into ``tiled_dense_gemm_mkl_amd/lib/libgemm_mkl.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libgemm_mkl.so")
OBJDIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
UNITS = ["gemm_api.hip", "inst_f32.hip", "inst_f16.hip", "inst_bf16.hip", "rms_norm.hip"]
HEADERS = ["gemm_kernels.hpp", "configs.hpp"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # no packed-fp32 VALU instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(unit: str) -> str:
    src = os.path.join(CSRC, unit)
    obj = os.path.join(OBJDIR, unit.replace(".hip", ".o"))
    cmd = [hipcc(), *common_flags(), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {unit}:\n{r.stderr[-4000:]}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every unit and link the shared library; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    jobs = jobs or min(len(UNITS), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, UNITS))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
