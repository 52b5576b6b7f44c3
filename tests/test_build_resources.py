"""Register and scratch use of every kernel in the built library, from the compiler's
kernel-resource-usage remarks that the build records beside librr.so (no GPU needed).  A
kernel that starts spilling to scratch memory after an edit fails here instead of silently
running slower."""
import json
import os

import pytest

from long_context_prefill_anchor_amd import build as B

# Kernels allowed to use scratch, with the most they may use (bytes per lane): the fp32-input
# reroute and fused relay instantiations, single and grouped (fp32 operands need twice the
# registers of bf16 at two waves per SIMD, and these carry the reroute's redo path too; the fp32
# workloads are the small 128- and 256-chunk ones).  The fp32 anchor / full-routing kernel runs
# without scratch.
SCRATCH_ALLOWED = {"k_routeIfLb0ELb1E": 80, "k_routeIfLb1ELb1E": 80,
                   "k_relayIfLb": 80, "k_relay_groupIfLb": 80}


@pytest.fixture(scope="module")
def usage():
    if not os.path.exists(B.RESOURCES):
        pytest.fail(f"{B.RESOURCES} is missing: build the library (python -m long_context_prefill_anchor_amd.build)")
    if os.path.getmtime(B.RESOURCES) + 1 < os.path.getmtime(B.LIB):
        pytest.fail("the resource report is older than librr.so: rebuild")
    with open(B.RESOURCES) as f:
        return json.load(f)


def test_report_covers_every_kernel_family(usage):
    names = " ".join(usage)
    for fam in ("k_route", "k_rescore", "k_relay", "k_compact_out", "k_route_wide", "k_sparse_attn"):
        assert fam in names, fam


def test_no_kernel_spills_to_scratch(usage):
    for name, u in usage.items():
        allowed = next((v for k, v in SCRATCH_ALLOWED.items() if k in name), 0)
        assert u["ScratchSize [bytes/lane]"] <= allowed, (name, u["ScratchSize [bytes/lane]"])
        assert u["VGPRs Spill"] == 0 or allowed > 0, (name, u["VGPRs Spill"])


def test_rescore_kernels_run_at_least_four_waves_per_simd(usage):
    """The relay rescoring is a gather: it needs many waves in flight per SIMD."""
    for name, u in usage.items():
        if "k_rescore" in name:
            assert u["Occupancy [waves/SIMD]"] >= 4, (name, u["Occupancy [waves/SIMD]"])


def test_parse_resource_remarks():
    lines = ["x.hip:1:1: remark: Function Name: _Z3foov [-Rpass-analysis=kernel-resource-usage]",
             "x.hip:1:1: remark:     VGPRs: 64 [-Rpass-analysis=kernel-resource-usage]",
             "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
             "x.hip:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]"]
    assert B.parse_resource_remarks(lines) == {"_Z3foov": {"VGPRs": 64, "ScratchSize [bytes/lane]": 0,
                                                          "Dynamic Stack": "False"}}
