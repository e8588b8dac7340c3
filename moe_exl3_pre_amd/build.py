"""Build the HIP library (gfx950) in-tree: moe_exl3_pre_amd/libexl3.so.

    python -m moe_exl3_pre_amd.build            # or: python moe_exl3_pre_amd/build.py

hipcc cross-compiles for gfx950 without a GPU present.  Packed-fp32 instruction selection is switched
off for the device code (those instructions are avoided on this hardware).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libexl3.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

SOURCES = ["exl3_api.cpp", "k_prepass.hip", "k_decode.hip", "k_gemm.hip", "k_moe.hip", "k_moe_tile.hip", "k_embed.hip", "k_mlp.hip", "k_probe.hip"]
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the EXL3 library)")


# Per-file code generation options.  The MoE kernels keep their MFMA accumulators in ordinary VGPRs
# (with the accumulator-register form the compiler splits the budget between the two files).  The
# prefill GEMM's 256 accumulators fill the accumulator file: the register-pressure-first scheduler keeps
# every MFMA accumulating in place (the default schedulers rename the results and copy them back each
# step).
EXTRA = {"k_moe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "k_gemm.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"],
         "k_moe_tile.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-minreg"]}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
