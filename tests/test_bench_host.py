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


def test_profile_summaries_round_trip(tmp_path, monkeypatch):
    """summarize_profiles turns rocprofv3 counter files into the committed summaries, and the
    bench reads them back only while the kernel source hash matches."""
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]

    def write(tag, rows):
        d = tmp_path / "runs" / tag
        d.mkdir(parents=True)
        lines = [",".join(cols)]
        for kname, grid, counter, value in rows:
            lines.append(",".join(["1", "1", "Agent 1", "1", "1", "1", str(grid), "1", f'"{kname}"', "512", "0", "0",
                                   "254", "0", "100", counter, str(value), "0", "1"]))
        (d / "pmc_counter_collection.csv").write_text("\n".join(lines) + "\n")

    relay = "void rr::k_relay<rr::bf16_t, false>(rr::RescoreArgs, rr::RouteArgs)"
    copy = "__amd_rocclr_copyBuffer"
    write("auto_util", [(relay, 131072, "SQ_ACTIVE_INST_VALU", 1000.0), (relay, 131072, "SQ_BUSY_CYCLES", 100.0),
                        (relay, 131072, "SQ_VALU_MFMA_BUSY_CYCLES", 320.0), (relay, 131072, "SQ_WAVES", 10.0),
                        (relay, 131072, "SQ_INSTS_VALU", 900.0)])
    write("auto_fetch", [(relay, 131072, "FETCH_SIZE", 4.0), (copy, 512, "FETCH_SIZE", 100.0),
                         (copy, 131072, "FETCH_SIZE", (bench.CALIB_BYTES >> 10) / 2)])
    write("auto_write", [(relay, 131072, "WRITE_SIZE", 2.0), (copy, 131072, "WRITE_SIZE", bench.CALIB_BYTES >> 10)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.txt"))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "counters.txt"))
    bench.summarize_profiles(str(tmp_path / "runs"), "rocprofv3 --pmc X -- python3 bench.py")
    # fetch counted at half the copy's bytes: scale 2; write scale 1
    assert bench.recorded_traffic("relay") == 4.0 * 1024 * 2 + 2.0 * 1024
    ctr = bench.recorded_counters("relay")
    assert abs(ctr["valu_busy"] - 1000.0 * 4 / (100.0 * 32)) < 1e-4
    assert abs(ctr["mfma_busy"] - 320.0 / (100.0 * 32)) < 1e-4
    assert ctr["valu_insts_per_wave"] == 90.0
    # a summary taken on other kernel sources is ignored
    text = (tmp_path / "traffic.txt").read_text().replace(bench.kernel_build_hash(), "0" * 64)
    (tmp_path / "traffic.txt").write_text(text)
    assert bench.recorded_traffic("relay") is None


def test_rho_breakdown_groups_layers_by_flagged_fraction():
    rho = [0.2, 0.3, 0.55, 0.9, 1.0]
    relay = np.array([[10.0, 20.0, 30.0, 40.0, 50.0], [12.0, 20.0, 30.0, 40.0, 50.0]]) / 1e3   # ms, 2 steps
    full = np.full((2, 5), 33.0) / 1e3
    out = bench.rho_breakdown(rho, relay, full)
    assert [b["rho"] for b in out] == [[0.0, 0.35], [0.5, 0.65], [0.8, 1.0]]
    assert [b["layers"] for b in out] == [2, 1, 2]
    first = out[0]
    assert first["relay_layer_us"] == 15.5 and first["full_layer_us"] == 33.0      # medians 11 and 20
    assert first["speedup_vs_full"] == round(33.0 / 15.5, 4) and first["rho_mean"] == 0.25
    assert out[2]["relay_layer_us"] == 45.0
