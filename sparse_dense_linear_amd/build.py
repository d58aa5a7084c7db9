"""Compile the HIP sources of this package (gfx950).

``libsdl_spmm.so`` is the library: each of its translation units is
compiled to an object under ``_build/`` (in parallel) and linked next to
this file.  ``libsdl_ceiling.so`` holds the measurement kernel that
``bench.py --gather-ceiling`` times (not part of the product path).
Packed fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libsdl_spmm.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "plan.hip", "worker.hip", "sddmm.hip", "eb.hip",
           "worker_f32_buf.hip", "worker_f32_flat.hip", "worker_bf16_buf.hip",
           "worker_bf16_flat.hip", "worker_fused_buf.hip", "worker_fused_flat.hip"]
CEILING_SOURCE = "ceiling.hip"
CEILING_PATH = os.path.join(HERE, "libsdl_ceiling.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    hipcc = _hipcc()
    flags = compile_flags()

    def one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, SOURCES + [CEILING_SOURCE]))
    for target, parts in ((LIB_PATH, objs[:-1]), (CEILING_PATH, objs[-1:])):
        tmp = target + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *parts]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed:\n{res.stderr}")
        os.replace(tmp, target)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
