"""Build librr.so (HIP for gfx950) in-tree with hipcc.

    python -m long_context_prefill_anchor_amd.build

All HIP code is compiled with packed-FP32 instructions disabled.
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
LIB = os.path.join(PKG, "librr.so")
SOURCES = ["rr_api.cpp", "rr_kernels.hip", "rr_attention.hip", "rr_wide.hip"]
ARCH = os.environ.get("RR_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def build(verbose: bool = False) -> str:
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # The route kernel runs two waves per SIMD (register-bound) and is latency-bound there;
           # the ILP-first scheduler spreads independent work between dependent instructions.
           "-mllvm", "-amdgpu-sched-strategy=max-ilp",
           # s_setprio around VALU-heavy stretches: the wave that holds the SIMD keeps issuing.
           "-mllvm", "-amdgpu-set-wave-priority",
           "-Wno-unused-command-line-argument",
           f"-I{INCLUDE}", f"-I{CSRC}"]
    cmd += ["-x", "hip"] + [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
