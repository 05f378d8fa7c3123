"""Builds the gfx950 HIP library libea02_attn.so in-tree with hipcc.

Usage: python -m exact_attention_02_amd.build   (or call build_library()).
Cross-compiles without a GPU.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libea02_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [os.path.join(CSRC, "attn_abi.hip"), os.path.join(CSRC, "attn_bwd.hip"),
           os.path.join(CSRC, "attn_mla.hip")]
DEPENDS = [os.path.join(CSRC, "attn_fwd_kernel.hpp"), os.path.join(CSRC, "attn_bwd_kernel.hpp"),
           os.path.join(CSRC, "attn_mla_kernel.hpp"),
           os.path.join(os.path.dirname(PKG_DIR), "include", "attn.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def build_library(verbose: bool = False, extra_flags=None) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), *SOURCES, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
