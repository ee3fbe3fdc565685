"""Build libpolykv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m quantized_shared_kv_amd.build

The library is written to quantized_shared_kv_amd/_lib/libpolykv.so.  Every
translation unit is compiled to its own object in parallel (``_lib/obj/``),
then linked.

    python -m quantized_shared_kv_amd.build --sanitize

builds a copy whose host code is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer (device code is built as usual) into
``_lib/san/libpolykv.so``.  Python is not instrumented, so the sanitizer
runtime must be loaded first; the host-only tests run against it with

    LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 PKV_LIBRARY=quantized_shared_kv_amd/_lib/san/libpolykv.so \
    python -m pytest tests/test_abi_host.py tests/test_handoff_host.py tests/test_comix_host.py  Every HIP translation unit is compiled with packed-fp32
instructions disabled, and matrix-core instructions write VGPRs
(-amdgpu-mfma-vgpr-form).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_lib")
OBJ_DIR = os.path.join(OUT_DIR, "obj")
LIB = os.path.join(OUT_DIR, "libpolykv.so")
SOURCES = ["pkv_host.cpp", "pkv_quantize.hip", "pkv_decode.hip", "pkv_decode_mfma.hip", "pkv_decode_mfma_split.hip",
           "pkv_comix.hip",
           "pkv_handoff.cpp", "pkv_stream.hip"]
SAN_DIR = os.path.join(OUT_DIR, "san")
ARCH = "gfx950"
# host-side sanitizers only: each -fsanitize= applies to the host compilation
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-fno-gpu-sanitize"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # matrix-core results in VGPRs: the score tiles are read by vector instructions, so
            # accumulating them in AGPRs cost a copy per value (the query operands sit in AGPRs)
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip())
    return r.returncode, errs


def build(verbose: bool = False, sanitize: bool = False) -> str:
    obj_dir = os.path.join(SAN_DIR, "obj") if sanitize else OBJ_DIR
    lib = os.path.join(SAN_DIR, "libpolykv.so") if sanitize else LIB
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    jobs = []
    for s in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [cc] + _flags() + extra + ["-c", "-o", obj, os.path.join(CSRC, s)]))
    if verbose:
        for _, cmd in jobs:
            print(" ".join(cmd), flush=True)
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda j: _run(j[1]), jobs))
    for (obj, _), (rc, errs) in zip(jobs, results):
        if rc != 0:
            raise RuntimeError(f"hipcc failed for {os.path.basename(obj)} ({rc}):\n{errs}")
        if verbose and errs:
            print(errs, flush=True)
    tmp = lib + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + (["-shared-libasan"] + extra if sanitize else []) + \
        ["-o", tmp] + [o for o, _ in jobs]
    if verbose:
        print(" ".join(link), flush=True)
    rc, errs = _run(link)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{errs}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
