"""Checks on the gfx950 assembly of the HIP kernels (CPU only: compiles, runs nothing).

The tile DMA is written as inline asm that loads M0 with the LDS destination
and issues global_load_lds_dwordx4.  M0 is a register the compiler may also
use for its own purposes; inline asm that clobbers it is only safe while the
compiler keeps nothing of its own in M0.  These tests compile each kernel
source to assembly and check that every M0 access in it is one of those
write + DMA pairs, so a compiler that starts using M0 fails here instead of
corrupting the kernels silently.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_diffusion_lm_td_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _asm(name, tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path / (name + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, name), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return [ln.split(";")[0].strip() for ln in out.read_text().splitlines()]


def _instructions(lines):
    return [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]


@pytest.mark.parametrize("name", ["td_attn.hip", "td_decode.hip", "td_commit.hip", "td_lmhead.hip",
                                  "td_append.hip", "td_mamba.hip", "td_adaln.hip"])
def test_m0_only_feeds_the_tile_dma(name, tmp_path):
    ins = _instructions(_asm(name, tmp_path))
    uses = [i for i, s in enumerate(ins) if re.search(r"\bm0\b", s)]
    for i in uses:
        s = ins[i]
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", s), f"M0 used outside the DMA pattern: {s!r}"
        assert ins[i + 1].startswith("global_load_lds_dwordx4"), \
            f"M0 write not followed by the DMA: {s!r} then {ins[i + 1]!r}"
    if name in ("td_attn.hip", "td_lmhead.hip"):
        assert uses, f"{name} should contain the tile DMA"

