"""Build libkda.so (gfx950 only) in-tree with hipcc.

    python -m gated_delta_rule_86_amd.build

Compiles csrc/kda_kernels.hip, csrc/kda_recurrent.hip, csrc/kda_noalloc.hip and
csrc/kda_backward.hip (device code) and csrc/kda_api.cpp (host C ABI) into
gated_delta_rule_86_amd/libkda.so.  Always rebuilds.
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
LIB = os.path.join(PKG, "libkda.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # keep MFMA accumulators in ordinary VGPRs (no accvgpr copies around VALU use)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, "kda_kernels.hip"), os.path.join(CSRC, "kda_recurrent.hip"),
            os.path.join(CSRC, "kda_noalloc.hip"), os.path.join(CSRC, "kda_backward.hip"),
            os.path.join(CSRC, "kda_api.cpp")]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("hipcc failed building libkda.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
