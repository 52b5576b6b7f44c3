"""Build librr.so (HIP for gfx950) in-tree with hipcc.

    python -m long_context_prefill_anchor_amd.build

All HIP code is compiled with packed-FP32 instructions disabled.
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librr.so")
# Per-kernel register, scratch, LDS and occupancy figures of the last build (the compiler's
# kernel-resource-usage remarks), written beside the library.
RESOURCES = os.path.join(PKG, "librr.resources.json")
# Measurement build: the same sources with phase timestamps compiled in (RR_PHASE_TRACE), for
# bench.py --phase-trace; never loaded by the library's users or tests.
PHASE_LIB = os.path.join(PKG, "librr_phase.so")
PHASE_RESOURCES = os.path.join(PKG, "librr_phase.resources.json")
SOURCES = ["rr_api.cpp", "rr_kernels.hip", "rr_attention.hip", "rr_wide.hip"]
ARCH = os.environ.get("RR_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found")
    return exe


def build(verbose: bool = False, phase_trace: bool = False) -> str:
    lib, resources = (PHASE_LIB, PHASE_RESOURCES) if phase_trace else (LIB, RESOURCES)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # The route kernel runs two waves per SIMD (register-bound) and is latency-bound there;
           # the ILP-first scheduler spreads independent work between dependent instructions.
           "-mllvm", "-amdgpu-sched-strategy=max-ilp",
           # s_setprio around VALU-heavy stretches: the wave that holds the SIMD keeps issuing.
           "-mllvm", "-amdgpu-set-wave-priority",
           "-Wno-unused-command-line-argument",
           # per-kernel VGPRs, scratch (spills), LDS and occupancy, parsed into RESOURCES
           "-Rpass-analysis=kernel-resource-usage",
           f"-I{INCLUDE}", f"-I{CSRC}"]
    if phase_trace:
        cmd.append("-DRR_PHASE_TRACE")
    cmd += ["-x", "hip"] + [os.path.join(CSRC, s) for s in SOURCES]
    tmp = lib + ".tmp"
    cmd += ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in res.stderr.splitlines() if noise not in l]
    remarks = [l for l in lines if "[-Rpass-analysis=kernel-resource-usage]" in l]
    err = "\n".join(l for l in lines if "-Rpass-analysis" not in l and not l.lstrip().startswith(("|", "^"))
                    and not re.match(r"^\s*\d+ \|", l))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    usage = parse_resource_remarks(remarks)
    with open(resources, "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    if verbose:
        for name, u in sorted(usage.items()):
            print(f"  {name}: VGPRs {u.get('VGPRs')} scratch {u.get('ScratchSize [bytes/lane]')} B/lane "
                  f"occupancy {u.get('Occupancy [waves/SIMD]')} waves/SIMD", flush=True)
    return lib


def parse_resource_remarks(lines):
    """{kernel symbol: {field: int}} from the compiler's kernel-resource-usage remarks."""
    out, cur = {}, None
    for line in lines:
        m = re.search(r"remark:\s+(.*?)\s+\[-Rpass-analysis", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            cur = text.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur is not None and ":" in text:
            key, val = text.rsplit(":", 1)
            val = val.strip()
            out[cur][key.strip()] = int(val) if val.lstrip("-").isdigit() else val
    return out


if __name__ == "__main__":
    print(build(verbose=True, phase_trace="--phase-trace" in sys.argv[1:]))
