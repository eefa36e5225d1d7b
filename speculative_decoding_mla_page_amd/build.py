"""Build libmla_verify.so in-tree with hipcc for gfx950.

Always recompiles; `python -m speculative_decoding_mla_page_amd.build` or
`build()` from Python.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmla_verify.so")
SOURCES = [os.path.join(PKG, "csrc", "mla_verify_api.cpp"),
           os.path.join(PKG, "csrc", "mla_verify_kernels.hip"),
           os.path.join(PKG, "csrc", "mla_verify_calibrate.hip"),
           os.path.join(PKG, "csrc", "mla_verify_noalloc.hip")]
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"),
    # no packed fp32 instructions in any generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep MFMA accumulators in VGPRs: the split-partial kernel's O accumulator
    # is rescaled in place, and the AGPR form makes the compiler copy it
    # between register files on every key tile
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # workgroup-wide counters (the device-side planner's per-request sums) reduce
    # each wave in DPP steps before its one atomic, instead of a scalar loop
    # over the active lanes
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=DPP",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-x", "hip", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
