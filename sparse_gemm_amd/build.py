"""Builds libbsr_linear.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m sparse_gemm_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libbsr_linear.so")
ARCH = "gfx950"

SOURCES = ["bsr_abi.cpp", "bsr_error.cpp", "bsr_pattern.cpp", "bsr_select.cpp", "bsr_kernels.hip", "bsr_wide.hip",
           "bsr_convert.hip", "bsr_fp8.hip", "bsr_sparse24.hip", "bsr_rebuild.hip"]
# Kernels whose 4 x 4 grids of 32 x 32 accumulators (256 registers per lane) must live in the
# accumulation registers: built without the flag that keeps accumulators in general registers.
AGPR_SOURCES = {"bsr_wide.hip"}

# Packed-fp32 instructions are kept out of the generated code on purpose; the host pass
# prints a harmless "not a recognized feature" warning for this flag.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form",   # MFMA accumulators stay in VGPRs (no AGPR copies)
             "-fno-gpu-rdc", f"-I{INCLUDE}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; always rebuilds."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        flags = [f for f in HIP_FLAGS if src not in AGPR_SOURCES or f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
        cmd = [hipcc()] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if res.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n" + "\n".join(noise))
        if noise and verbose:
            print("\n".join(noise), file=sys.stderr)
        return obj

    jobs = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 8))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
