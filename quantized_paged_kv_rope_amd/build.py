"""Compile the gfx950 HIP library ``libkvrec.so`` in-tree with hipcc.

Flags that matter for bit-exact results:
  -ffp-contract=off                no fused multiply-add anywhere (the RoPE is
                                   two rounded products and one rounded add)
  -fno-gpu-flush-denormals-to-zero fp32 denormals kept (inputs and results)
  -target-feature -packed-fp32-ops no v_pk_{add,mul,fma}_f32 generated
Performance flag:
  -amdgpu-kernarg-preload-count=16 kernel arguments arrive in SGPRs
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libkvrec.so")
ARCH = "gfx950"

SOURCES = ["kvrec_kernels.hip", "kvrec_expand.hip", "kvrec_api.cpp"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # gfx950 loads the leading kernel arguments into SGPRs at wave launch
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)  # host pass: feature is device-only
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libkvrec.so``; returns its path."""
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        _run([hipcc(), *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def device_asm(verbose: bool = False) -> str:
    """gfx950 assembly of the kernels (for the no-FMA / no-packed-fp32 check)."""
    out = os.path.join(PKG, "_build", "kvrec_kernels.gfx950.s")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    _run([hipcc(), *COMMON_FLAGS, "-x", "hip", "--cuda-device-only", "-S",
          os.path.join(CSRC, "kvrec_kernels.hip"), "-o", out], verbose)
    with open(out) as f:
        return f.read()


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
