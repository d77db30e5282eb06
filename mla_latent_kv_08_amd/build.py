"""Build libmla.so (HIP for gfx950) in-tree with hipcc.

Usage: python -m mla_latent_kv_08_amd.build [--asm]
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # Keep the compiler from forming packed fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-op accumulators in VGPRs: the attention kernel's O accumulators
    # then stay put across the tile loop (no AGPR<->VGPR copies each tile),
    # and its query fragments sit in AGPRs, which the matrix ops read directly.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "mla_api.cpp")]


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    """Compile every HIP source and the C ABI into libmla.so; returns its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC, "-o", tmp, *sources()]
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps=cwd", "-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=asm_dir or PKG, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose or asm_dir:
        sys.stderr.write(res.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    asm = None
    if "--asm" in sys.argv:
        asm = os.path.join(ROOT, "_build", "asm")
    print(build(verbose=True, asm_dir=asm))
