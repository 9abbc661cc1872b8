"""Build libtdm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m tiled_dense_matrix_amd.build   (or call ``build()``)

Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so it travels with the source tree.
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
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "tdm")
LIB = os.path.join(PKG, "libtdm.so")

ARCH = "gfx950"
SOURCES = [
    "tdm_api.hip",
    "gemm_edge.hip",
    "gemm_valu_f32.hip",
    "gemm_mfma_bf16.hip",
    "gemm_mfma_f32.hip",
    "gemm_skinny_bf16.hip",
    "gemm_skinny_nk_bf16.hip",
    "gemm_mfma_fp8.hip",
    "attention_fwd.hip",
]

# Packed fp32 instructions are switched off for all device code: the kernels
# are written for single fp32 FMAs and the matrix cores.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXXFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
            "-Wno-unused-command-line-argument", "-fvisibility=hidden", f"-I{INCLUDE}", f"-I{CSRC}"] + DEVICE_FLAGS


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libtdm.so")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libtdm.so. Always rebuilds."""
    os.makedirs(OBJDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
