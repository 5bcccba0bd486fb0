"""Build libpda.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m decode_attention_fp8_write_amd.build [--save-temps DIR]
"""
from __future__ import annotations

import argparse
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpda.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off for every HIP source.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # matrix-core products the compiler places write VGPRs: the
                # latent kernel's score tiles stay out of the AGPRs its inline-asm
                # output accumulators fill
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(
        glob.glob(os.path.join(CSRC, "*.cpp")))


def build(save_temps: str | None = None, verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function",
           # a pointer squeezed through a 32-bit value (e.g. a lane broadcast
           # builtin that takes int) is an address fault on the GPU: refuse it
           "-Werror=int-to-pointer-cast", "-Werror=pointer-to-int-cast",
           "-Werror=shorten-64-to-32",
           *DEVICE_FLAGS, "-I", INCLUDE, "-I", CSRC,
           "-o", tmp, *sources()]
    cwd = None
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "-save-temps")
        cwd = save_temps
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=cwd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--save-temps", default=None)
    args = ap.parse_args()
    print(build(args.save_temps, verbose=True))
    sys.exit(0)
