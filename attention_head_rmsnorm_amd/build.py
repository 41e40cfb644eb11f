"""Builds libflint_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m attention_head_rmsnorm_amd.build`` (or ``build()`` from
Python). The library lands next to this file, where the binding loads it.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SRCS = [os.path.join(CSRC, f) for f in ("flint_attn.hip", "flint_decode.hip", "flint_bwd.hip", "flint_bshd.hip", "flint_proj.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libflint_attn.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", INCLUDE, *SRCS, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
