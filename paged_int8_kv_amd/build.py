"""Build libkv8.so (the HIP library) in-tree with hipcc for gfx950.

    python -m paged_int8_kv_amd.build

Objects go to paged_int8_kv_amd/_build/, the library to
paged_int8_kv_amd/_lib/libkv8.so.  No GPU is needed: hipcc cross-compiles.
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
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libkv8.so")

ARCH = "gfx950"
SOURCES = ["kv8_api.cpp", "kv8_append.hip", "kv8_decode.hip", "kv8_decode_mfma.hip",
           "kv8_decode_sk.hip", "kv8_prefill.hip", "kvbf16_decode.hip", "kv8_probe.hip"]

# Packed fp32 VALU instructions are kept out of the code object: the
# compiler's automatic use of them is switched off for every HIP source.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]

# Per-source extra flags.  The MFMA kernels keep their accumulators in
# ordinary VGPRs: with the accumulator-register form the compiler copied all
# 128 prefill accumulators between register files on every key tile, and the
# matrix-core decode needs 96 VGPRs in one file (5 waves per SIMD) against
# 96 + 36 split over two (3 waves).
EXTRA_FLAGS = {
    "kv8_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    "kv8_decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
    "kv8_decode_sk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}


def hipcc_path():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libkv8")


def _compile(hipcc, src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libkv8.so; returns the library path."""
    hipcc = hipcc_path()
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s, verbose), SOURCES))
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
