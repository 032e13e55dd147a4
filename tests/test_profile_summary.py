"""CPU checks of the profile summaries (tree_verify_mla_attn_amd/profile_summary.py) on
small synthetic rocprofv3 outputs: the trace's per-step phase span and fraction, the
counter calibration against the copy, and the bench-line table."""
import csv
import json

import pytest

from tree_verify_mla_attn_amd import profile_summary as PS

LINE = {"value": 1.0, "ms_per_step": 1.0, "steps_per_s": 1000.0, "dtype": "bf16 in",
        "config": {"workload": "w", "num_splits": 1, "algorithmic_flops": 2.5e9,
                   "algorithmic_bytes": 1_000_000},
        "roofline": {"kernel": "attention", "achieved": 2.5, "peak": 2500.0, "frac": 0.001},
        "hbm": {"frac": 0.1, "call_bytes_over_algorithmic": 2.0},
        "cpu_baseline": {"value": 0.3}}


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=header)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_trace_phase_span_and_fraction(tmp_path):
    # two steps; each: pre-pass, then attention 1000..2000 ns after a 100 ns gap
    rows = []
    for step in range(2):
        t0 = step * 10_000
        rows.append({"Kernel_Name": "prepass_kernel(x)", "Start_Timestamp": t0,
                     "End_Timestamp": t0 + 500})
        rows.append({"Kernel_Name": "verify_attn_bf16_kernel(x)", "Start_Timestamp": t0 + 600,
                     "End_Timestamp": t0 + 1600})
    (tmp_path / "kt").mkdir()
    _write_csv(tmp_path / "kt" / "kt_kernel_trace.csv",
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    (tmp_path / "b.log").write_text("noise\n" + json.dumps(LINE) + "\n")
    out = PS.trace(str(tmp_path / "kt"), str(tmp_path / "b.log"), 0, 2, "cmd")
    # 2.5e9 flop in 1 us = 2500 TFLOP/s = frac 1.0 of 2500
    assert "1.00 us per call" in out and "1.0000 of 2500 TFLOP/s" in out
    assert "trace / line = 1000.0000" in out


def test_counters_scaled_by_the_calibration_copy(tmp_path, monkeypatch):
    def run(counter, kib_attn, kib_copy):
        rows = [{"Dispatch_Id": 1, "Kernel_Name": "verify_attn_bf16_kernel", "Counter_Name": counter,
                 "Counter_Value": kib_attn},
                {"Dispatch_Id": 2, "Kernel_Name": "prepass_kernel", "Counter_Name": counter,
                 "Counter_Value": 10.0},
                {"Dispatch_Id": 3, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                 "Counter_Value": kib_copy}]
        p = tmp_path / f"{counter}.csv"
        _write_csv(p, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
        return str(p)
    monkeypatch.setattr(PS, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    # the 256 MiB copy reads half its bytes on FETCH_SIZE (factor 2), all on WRITE_SIZE
    entry = PS.traffic(run("FETCH_SIZE", 1000.0, 131072.0), run("WRITE_SIZE", 500.0, 262144.0),
                       "w", 1, 4, ["c1", "c2"])
    assert entry["fetch_copy_factor"] == pytest.approx(2.0)
    assert entry["write_copy_factor"] == pytest.approx(1.0)
    assert entry["kernels"]["verify_attn_bf16_kernel"] == {"fetch_kib": 1000.0, "write_kib": 500.0,
                                                           "dispatches": 1}
    text = PS.traffic_text(entry, LINE)
    # phase: 2000 KiB fetched + 500 KiB written = 2.56 MB, of 1 MB algorithmic
    assert "2.0 MB fetched + 0.5 MB written = 2.6 MB (2.56x" in text
    stored = json.load(open(tmp_path / "traffic.json"))["entries"]
    assert len(stored) == 1 and stored[0]["workload"] == "w"


def test_bench_table_rows(tmp_path):
    d = tmp_path / "box"
    d.mkdir()
    for w in (1, 4):
        line = dict(LINE, config=dict(LINE["config"], workload=f"w{w}"))
        (d / f"bench_w{w}.log").write_text(json.dumps(line) + "\n")
    out = PS.bench_table([str(d)])
    rows = [r for r in out.splitlines() if r.startswith("| 1 |") or r.startswith("| 4 |")]
    assert len(rows) == 2 and "| w4 |" in rows[1] and "| 2.0 |" in rows[1]
