"""Host-side pieces of bench.py: the recall metric, the fixed-stride baseline, the one-GPU
rule and the traffic record's source check (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_route_recall_counts_overlap_per_row():
    exact = np.array([[0, 1, 2, 3], [4, 5, 6, 7]])
    used = np.array([[3, 2, 9, 8], [4, 5, 6, 7]])          # row 0: 2 of 4, row 1: 4 of 4
    assert bench.route_recall(used, exact) == 0.75


def test_route_recall_ignores_padding():
    exact = np.array([[0, 1, -1, -1]])                      # a short (causal) row: 2 real entries
    used = np.array([[1, -1, -1, 5]])                       # -1 in used never matches a real entry
    assert bench.route_recall(used, exact) == 0.5
    assert bench.route_recall(exact, exact) == 1.0


def test_stride_reuse_refreshes_every_fourth_layer():
    exact = [np.full((2, 3), l) for l in range(9)]
    used = bench.stride_reuse_routes(exact, 4)
    assert [int(u[0, 0]) for u in used] == [0, 0, 0, 0, 4, 4, 4, 4, 8]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_traffic_record_needs_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    """The committed counter summary is used only while the hash of the routing kernel source,
    its headers and the build script matches the one written in it; any change to those files
    (here: one more byte in a copy of the source) turns the traffic figure into None."""
    good = bench.kernel_build_hash()
    src = tmp_path / "rr_kernels.hip"
    src.write_bytes(open(bench.KERNEL_SRCS[0], "rb").read() + b"\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", (str(src),) + tuple(bench.KERNEL_SRCS[1:]))
    assert bench.kernel_build_hash() != good
    assert bench.recorded_traffic("reroute") is None
    assert any(p.endswith("rr_device.h") for p in bench.KERNEL_SRCS)
