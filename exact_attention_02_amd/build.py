"""Builds the gfx950 HIP library libea02_attn.so in-tree with hipcc.

Usage: python -m exact_attention_02_amd.build   (or call build_library()).
Cross-compiles without a GPU.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libea02_attn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = [os.path.join(CSRC, "attn_abi.hip"), os.path.join(CSRC, "attn_bwd.hip"),
           os.path.join(CSRC, "attn_mla.hip")]
DEPENDS = [os.path.join(CSRC, "attn_fwd_kernel.hpp"), os.path.join(CSRC, "attn_bwd_kernel.hpp"),
           os.path.join(CSRC, "abi_util.hpp"),
           os.path.join(CSRC, "attn_mla_kernel.hpp"),
           os.path.join(os.path.dirname(PKG_DIR), "include", "attn.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source flags.  The backward was built with -mllvm
# -amdgpu-mfma-vgpr-form while its dK/dV accumulators were inline-asm MFMAs on
# AGPRs; with every MFMA a builtin, the compiler's own placement
# (accumulators in AGPRs) measured faster than that flag's VGPR form.
# The backward's kernels are scheduled with the machine scheduler's
# memory-clause strategy: 0.4-0.6 % faster whole backward than the default
# (causal GQA-4 N=8192-32768, GQA-8 N=4096), bit-identical gradients.  The
# forward measured 1-2 % slower with it and keeps the default.
SOURCE_FLAGS: dict = {"attn_bwd.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _check(r, cmd, verbose):
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build_library(verbose: bool = False, extra_flags=None) -> str:
    """Compile each source to an object (in parallel), then link."""
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="ea02_build_") as d:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = [hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []),
                   *(extra_flags or []), "-c", src, "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                                text=True)))
            objs.append(obj)
        for cmd, pr in procs:
            out, err = pr.communicate()
            _check(subprocess.CompletedProcess(cmd, pr.returncode, out, err), cmd, verbose)
        cmd = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", *objs, "-o", tmp]
        _check(subprocess.run(cmd, capture_output=True, text=True), cmd, verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
