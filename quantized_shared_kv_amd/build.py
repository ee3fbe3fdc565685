"""Build libpolykv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m quantized_shared_kv_amd.build

The library is written to quantized_shared_kv_amd/_lib/libpolykv.so.  Every
HIP translation unit is compiled with packed-fp32 instructions disabled, and
matrix-core instructions write VGPRs (-amdgpu-mfma-vgpr-form).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "libpolykv.so")
SOURCES = ["pkv_host.cpp", "pkv_quantize.hip", "pkv_decode.hip", "pkv_decode_mfma.hip", "pkv_comix.hip", "pkv_handoff.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # matrix-core results in VGPRs: the score tiles are read by vector instructions, so
           # accumulating them in AGPRs cost a copy per value (the query operands sit in AGPRs)
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{errs}")
    if verbose and errs:
        print(errs, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
