"""bench.py's host-side parts, on the CPU: the one-GPU guard, the
algorithmic work model, the rocprofv3 summary helper and the traffic
record's staleness check."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from sparse_moe_transformer_fp32_amd.inputs import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_layer_work_flash_prefill_closed_form():
    """Every expert touched at T=4096: 1.160e12 bf16 FLOPs per layer (two
    gated-FFN passes of 3 H x I matrices over K T routed rows and T shared
    rows) and 9.16 GB of weights, router, x and y."""
    wl = WORKLOADS["prefill"]
    w = bench.layer_work(wl, np.full(wl.E, 114))
    T, H, E, K, I = 4096, 4096, 288, 8, 1280
    assert w["n_active"] == E
    assert w["layer_flops"] == 2 * 3 * H * I * (K * T + T)
    assert abs(w["layer_flops"] - 1.160e12) < 1e9
    assert w["gu_flops"] == 2 * 2 * H * I * (K * T + T)
    assert w["layer_bytes"] == 3 * H * I * 2 * (E + 1) + E * H * 4 + E * 4 + 2 * T * H * 2
    assert abs(w["layer_bytes"] - 9.16e9) < 0.01e9


def test_layer_work_counts_only_active_experts():
    wl = WORKLOADS["decode"]
    counts = np.zeros(wl.E, dtype=np.int64)
    counts[[3, 10, 200]] = [100, 27, 1]
    w = bench.layer_work(wl, counts)
    assert w["n_active"] == 3
    per_expert = 3 * wl.H * wl.I * 2
    assert w["layer_bytes"] - (4 * per_expert) == wl.E * wl.H * 4 + wl.E * 4 + 2 * wl.T * wl.H * 2


def _write_csv(path, header, rows):
    with open(path, "w") as f:
        f.write(",".join(f'"{h}"' for h in header) + "\n")
        for r in rows:
            f.write(",".join(f'"{v}"' for v in r) + "\n")


def test_summarize_stats_splits_launch_shapes(tmp_path):
    stats = tmp_path / "stats.csv"
    _write_csv(stats, ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"],
               [["smoe::k_a", 3, 900000, 300000, 100000, 400000],
                ["other_kernel", 1, 5, 5, 5, 5]])
    trace = tmp_path / "trace.csv"
    hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X",
           "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    _write_csv(trace, hdr, [["smoe::k_a", 0, 400000, 256, 1, 1, 256 * 100, 1, 1],
                            ["smoe::k_a", 0, 400000, 256, 1, 1, 256 * 100, 1, 1],
                            ["smoe::k_a", 0, 100000, 64, 1, 1, 64 * 16, 5, 2],
                            ["other_kernel", 0, 5, 1, 1, 1, 1, 1, 1]])
    out = tmp_path / "summary.txt"
    bench.summarize_stats(str(stats), str(out), "the command", str(trace))
    text = out.read_text()
    assert "# command: the command" in text
    assert "other_kernel" not in text
    lines = [l.split() for l in text.splitlines() if l and not l.startswith("#")]
    # the per-kernel row, then one row per launch shape: (calls, avg, min, max, wgs)
    shape_rows = [l for l in lines if len(l) == 6 and l[4].isdigit()]
    got = sorted((int(l[0]), float(l[1]), int(l[4])) for l in shape_rows)
    assert got == [(1, 100.0, 160), (2, 400.0, 100)]


def test_traffic_record_goes_stale_with_its_sources(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "decode", ["kernel.hip"])
    (tmp_path / "profiles").mkdir()
    rec = {"gate_up:decode": {"bytes_per_launch": 12345,
                              "source_sha": bench._src_sha(["kernel.hip"])}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench._traffic("gate_up:decode") == 12345
    src.write_text("kernel v2\n")
    assert bench._traffic("gate_up:decode") is None
    assert bench._traffic("gate_up:prefill") is None


def test_summarize_mfma_derived_columns(tmp_path):
    """MFMA work = MOPS x 512, clock = GRBM_GUI_ACTIVE / 8 over the dispatch
    time, busy = MFMA busy cycles over 1024 SIMDs x cycles."""
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
           "End_Timestamp"]
    for wl in ("prefill", "long"):
        (tmp_path / wl).mkdir()
        rows = []
        for disp, kern in ((1, "void smoe::expert_gemm_lds_kernel<0>(P)"),
                           (2, "void smoe::expert_gemm_lds_kernel<1>(P)")):
            cycles = 2_000_000                      # per XCD: 1 ms at 2 GHz
            vals = {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e9 / 512,
                    "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 1024 * cycles, "SQ_LDS_BANK_CONFLICT": 7,
                    "SQ_WAVES": 64, "SQ_BUSY_CU_CYCLES": 1, "SQ_LDS_IDX_ACTIVE": 1,
                    "SQ_WAVE_CYCLES": 1}
            for c, v in vals.items():
                rows.append([disp, kern, c, v, 0, 1_000_000])
        _write_csv(tmp_path / wl / "run_counter_collection.csv", hdr, rows)
    lines = bench.summarize_mfma(str(tmp_path), "the command")
    assert "#   the command" in lines
    data = [l.split() for l in lines if l.startswith(("prefill", "long"))]
    assert len(data) == 4
    for wl, kernel, t_us, clock, mfma_tf, alg_tf, pad, busy, conf, waves in data:
        assert float(t_us) == 1000.0 and float(clock) == 2.0
        assert float(mfma_tf) == 0.001 and busy == "25.0%" and conf == "7" and waves == "64"
        w = WORKLOADS[wl]
        alg = 2 * (w.K * w.T * 2 * w.I * w.H + w.T * 2 * w.Is * w.H) / (1 if kernel == "gate_up" else 2)
        assert abs(float(alg_tf) - alg / 1e12) < 1e-3
