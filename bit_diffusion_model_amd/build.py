"""Build libsvdq.so in-tree: HIP kernels for gfx950 plus the host C++ pack.

Usage: python -m bit_diffusion_model_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsvdq.so")
BUILD = os.path.join(HERE, "_build")
ARCH = "gfx950"

DEVICE_SOURCES = ["k1_quant_lora_down.hip", "k2_gemm_w4a4.hip", "k3_lora_up.hip", "k4_w4a16.hip", "api.cpp", "noalloc.hip"]
HOST_SOURCES = ["pack.cpp", "status.cpp"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU ops stay disabled on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-march=x86-64-v3", "-ffp-contract=off",
              "-fno-fast-math", "-pthread"]


def _hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _host_cxx() -> str:
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("g++") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("no host C++ compiler found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link libsvdq.so next to this file. Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc, cxx = _hipcc(), _host_cxx()
    jobs = []
    for s in DEVICE_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append([hipcc, *HIP_FLAGS, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o])
    for s in HOST_SOURCES:
        o = os.path.join(BUILD, s + ".o")
        jobs.append([cxx, *HOST_FLAGS, "-I", CSRC, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=4) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr)
    objs = [os.path.join(BUILD, s + ".o") for s in DEVICE_SOURCES + HOST_SOURCES]
    tmp = OUT + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    p = build(verbose="-v" in sys.argv)
    print(p)
