"""Build libspecverify.so (gfx950) in-tree with hipcc.

    python -m lossless_draft_verification_row_amd.build

The library lands next to this file.  Every call rebuilds it from the sources.
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
LIB_NAME = "libspecverify.so"
SOURCES = ["spec_api.hip", "spec_kernels.hip", "spec_fused.hip", "spec_filter.hip", "spec_head.hip",
           "spec_noalloc.hip"]
ARCH = os.environ.get("SPEC_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libspecverify")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 vector ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose=False) -> str:
    out = os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), *compile_flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
