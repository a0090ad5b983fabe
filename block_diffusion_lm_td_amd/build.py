"""Build libtd.so in-tree for gfx950 (hipcc for the kernels, g++ for the
HIP-free host code).  ``python -m block_diffusion_lm_td_amd.build``."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtd.so")
BUILD = os.path.join(ROOT, "_build")

HIP_SOURCES = ["td_attn.hip", "td_decode.hip", "td_commit.hip", "td_lmhead.hip", "td_mamba.hip", "td_adaln.hip", "td_append.hip", "td_noalloc.hip"]
HOST_SOURCES = ["td_plan.cpp", "td_api.cpp"]
ARCH = "gfx950"
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
               # packed fp32 VALU forms stay disabled on this target
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libtd.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile every source and link libtd.so into the package directory."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run([hipcc, *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
