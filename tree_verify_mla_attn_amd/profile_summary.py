"""Summaries of rocprofv3 output for the committed profiles.

    python -m tree_verify_mla_attn_amd.profile_summary trace  KT_DIR BENCH_LOG WARMUP STEPS CMD
    python -m tree_verify_mla_attn_amd.profile_summary traffic FETCH_CSV WRITE_CSV WORKLOAD SPLITS CALLS CMD1 CMD2
    python -m tree_verify_mla_attn_amd.profile_summary traffic-text WORKLOAD SPLITS BENCH_LOG
    python -m tree_verify_mla_attn_amd.profile_summary counters CSV CMD
    python -m tree_verify_mla_attn_amd.profile_summary bench-table DIR [DIR ...]
    python -m tree_verify_mla_attn_amd.profile_summary greedy-trace KT_DIR BENCH_LOG CMD

`trace` reads a --kernel-trace --stats run of bench.py (its kernel trace CSV and the JSON
line the same run printed) and recomputes the roofline fraction from the traced kernel
durations of the timed steps.  `traffic` reads one FETCH_SIZE and one WRITE_SIZE counter
run of bench.py --calibrate-copy, scales each counter by what it reads for the 256 MiB
calibration copy, and merges the per-kernel bytes into profiles/traffic.json, where
bench.py finds them; `traffic-text` prints one stored entry beside the algorithmic bytes
of the workload's bench line.  `counters` prints per-kernel means of any other counter run.
`bench-table` tabulates the JSON lines of `bench.py --workload W` runs (W = 1..5, logged
as DIR/bench_wW.log), one table per DIR (one box each).  `greedy-trace` reads a kernel
trace of a default bench.py run (greedy step included) and summarises the builder, pack,
accept and draw kernels.
"""
from __future__ import annotations

import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")

# The kernels of one kdtree_verify_attn call, and the ones the attention phase (the
# roofline's kernel) covers: everything after the pre-pass.
CALL_KERNELS = ("prepass_kernel", "fill_nan_kernel", "verify_attn_bf16_kernel",
                "verify_attn_f32_kernel", "piece_merge_kernel", "lse_merge_kernel")
PHASE_KERNELS = CALL_KERNELS[1:]
CALIBRATION_BYTES = 256 << 20   # bench.py --calibrate-copy: one 256 MiB device copy


def short_name(full: str) -> str:
    for k in CALL_KERNELS:
        if k in full:
            return k
    return full.split("(")[0][:60]


def bench_line(path: str) -> dict:
    lines = [ln for ln in open(path).read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1])


def trace(kt_dir: str, bench_log: str, warmup: int, steps: int, cmd: str) -> str:
    rows = list(csv.DictReader(open(os.path.join(kt_dir, "kt_kernel_trace.csv"))))
    per = defaultdict(list)
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        name = short_name(r["Kernel_Name"])
        if name in CALL_KERNELS:
            per[name].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    line = bench_line(bench_log)
    # the timed steps: dispatches warmup .. warmup + steps - 1 of each kernel of the call
    # (the cut's fill + piece merge run once per call, like the attention kernel)
    spans = {k: v[warmup:warmup + steps] for k, v in per.items() if len(v) >= warmup + steps}
    timed = {k: [(e - b) / 1e3 for b, e in v] for k, v in spans.items()}
    # the attention phase of step i: first start to last end of its kernels (the launch
    # gaps between them included, as the HIP events around the phase include them)
    phase = [k for k in spans if k in PHASE_KERNELS]
    step_us = [(max(spans[k][i][1] for k in phase) - min(spans[k][i][0] for k in phase)) / 1e3
               for i in range(steps)]
    phase_us = sum(step_us) / steps
    busy_us = sum(sum(v) / len(v) for k, v in timed.items() if k in PHASE_KERNELS)
    flops = line["config"]["algorithmic_flops"]
    peak = line["roofline"]["peak"]
    frac = flops / (phase_us * 1e-6) / 1e12 / peak
    out = [f"# rocprofv3 kernel trace: {line['config']['workload']}, "
           f"num_splits {line['config']['num_splits']}",
           "",
           "Command (from the repository root, on one MI355X; rocprofv3 run from /tmp with "
           "TMPDIR=/tmp):",
           f"  {cmd}",
           "",
           f"Per kernel of the call, the {steps} timed steps (dispatches {warmup}.."
           f"{warmup + steps - 1} in time order):",
           "  kernel | dispatches | avg us | min us | max us"]
    for k in CALL_KERNELS:
        if k in timed:
            v = timed[k]
            out.append(f"  {k} | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f}")
    out += ["",
            f"Attention phase ({line['roofline']['kernel']}): {phase_us:.2f} us per call from the "
            f"trace (first start to last end of its kernels; {busy_us:.2f} us of kernel time) -> "
            f"{flops / (phase_us * 1e-6) / 1e12:.1f} TFLOP/s, {frac:.4f} of {peak:.0f} TFLOP/s.",
            f"The same run's bench line: achieved {line['roofline']['achieved']} TFLOP/s, frac "
            f"{line['roofline']['frac']} (HIP events around the phase on its stream); "
            f"trace / line = {frac / line['roofline']['frac']:.4f}.",
            "",
            "Bench line of the run:",
            "  " + json.dumps(line)]
    return "\n".join(out) + "\n"


def _per_kernel(csv_path: str, counter: str, calls: int):
    """Mean counter value per kernel over its first `calls` dispatches (the warm-up and
    timed calls of the workload; bench.py may launch other shapes after them), and the
    largest device-copy reading (the calibration copy)."""
    vals = defaultdict(list)
    copies = []
    rows = [r for r in csv.DictReader(open(csv_path)) if r["Counter_Name"] == counter]
    for r in sorted(rows, key=lambda r: int(r["Dispatch_Id"])):
        name, v = short_name(r["Kernel_Name"]), float(r["Counter_Value"])
        if "copyBuffer" in r["Kernel_Name"]:
            copies.append(v)
        vals[name].append(v)
    means = {k: sum(v[:calls]) / len(v[:calls]) for k, v in vals.items()}
    return means, {k: len(v[:calls]) for k, v in vals.items()}, max(copies) if copies else None


def traffic(fetch_csv: str, write_csv: str, workload: str, splits: int, calls: int,
            cmds) -> dict:
    sys.path.insert(0, ROOT)
    import bench
    fetch, n_f, copy_f = _per_kernel(fetch_csv, "FETCH_SIZE", calls)
    write, n_w, copy_w = _per_kernel(write_csv, "WRITE_SIZE", calls)
    ff = CALIBRATION_BYTES / (copy_f * 1024)
    wf = CALIBRATION_BYTES / (copy_w * 1024)
    kernels = {k: {"fetch_kib": round(fetch[k], 1), "write_kib": round(write.get(k, 0.0), 1),
                   "dispatches": n_f[k]}
               for k in CALL_KERNELS if k in fetch}
    entry = {"workload": workload, "num_splits": splits,
             "kernel_source_sha256": bench.kernel_source_digest(),
             "fetch_copy_factor": round(ff, 5), "write_copy_factor": round(wf, 5),
             "calibration_copy_kib": {"fetch": copy_f, "write": copy_w},
             "kernels": kernels, "commands": list(cmds)}
    try:
        doc = json.load(open(TRAFFIC_JSON))
        entries = doc.get("entries", [])
    except (OSError, ValueError):
        entries = []
    entries = [e for e in entries if not (e.get("workload") == workload and
                                          e.get("num_splits") == splits)]
    entries.append(entry)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump({"entries": entries}, f, indent=1)
        f.write("\n")
    return entry


def traffic_text(entry: dict, line: dict) -> str:
    """The per-kernel HBM bytes of one traffic.json entry as a text summary, beside the
    call's algorithmic bytes (from the bench line of the workload)."""
    ff, wf = entry["fetch_copy_factor"], entry["write_copy_factor"]
    alg = line["config"]["algorithmic_bytes"]
    out = [f"# HBM traffic counters: every kernel of one call, workload {entry['workload']}, "
           f"num_splits {entry['num_splits']}",
           "",
           "Commands (from the repository root, one counter per pass, each its own run; "
           "rocprofv3 run from /tmp with TMPDIR=/tmp):"]
    out += [f"  {c}" for c in entry["commands"]]
    cf, cw = entry["calibration_copy_kib"]["fetch"], entry["calibration_copy_kib"]["write"]
    out += ["",
            "Calibration: bench.py --calibrate-copy ends with one 256 MiB device-to-device copy",
            f"  FETCH_SIZE of the copy = {cf:.1f} KiB -> factor {ff:.5f} (true bytes / counter bytes)",
            f"  WRITE_SIZE of the copy = {cw:.1f} KiB -> factor {wf:.5f}",
            "",
            "Per dispatch (mean over the workload's warm-up and timed calls), scaled by those "
            "factors:",
            "  kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB"]
    tf = tw = pf = pw = 0.0
    for k, v in entry["kernels"].items():
        f, w = v["fetch_kib"] * ff * 1024 / 1e6, v["write_kib"] * wf * 1024 / 1e6
        out.append(f"  {k} | {v['fetch_kib']:.1f} | {v['write_kib']:.1f} | {f:.1f} | {w:.1f}")
        tf, tw = tf + f, tw + w
        if k in PHASE_KERNELS:
            pf, pw = pf + f, pw + w
    out += ["",
            f"Attention phase ({line['roofline']['kernel']}): {pf:.1f} MB fetched + {pw:.1f} MB "
            f"written = {pf + pw:.1f} MB ({(pf + pw) * 1e6 / alg:.2f}x the algorithmic bytes).",
            f"Whole call (pre-pass included): {tf:.1f} MB fetched + {tw:.1f} MB written = "
            f"{tf + tw:.1f} MB ({(tf + tw) * 1e6 / alg:.2f}x).",
            f"Algorithmic bytes of the call (Q, K and V once at input precision, fp32 output "
            f"+ lse): {alg / 1e6:.1f} MB.",
            f"Kernel sources: sha256 {entry['kernel_source_sha256']}"]
    return "\n".join(out) + "\n"


def counters(csv_path: str, cmd: str) -> str:
    per = defaultdict(lambda: defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        per[short_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = [f"Command: {cmd}", "  kernel | counter | dispatches | mean"]
    for k in CALL_KERNELS:
        for c, v in sorted(per.get(k, {}).items()):
            out.append(f"  {k} | {c} | {len(v)} | {sum(v) / len(v):.6g}")
    return "\n".join(out) + "\n"


def bench_table(dirs) -> str:
    out = ["# bench.py lines of the five workloads (defaults), one MI355X per table",
           "",
           "Command, from the repository root, one run per workload, back to back on one box:",
           "  python3 bench.py --workload W          (W = 1..5; W = 4 is the default)",
           "",
           "value = algorithmic TFLOP/s of the whole call (pre-pass + attention + merge) from the",
           "wall clock around the timed steps; frac = the attention phase (the roofline kernel",
           "column) from HIP events on its stream, over the dtype's dense MFMA peak (bf16 path:",
           "2500 TFLOP/s; fp32 path: 157.3); HBM frac = algorithmic bytes over the phase time",
           "against 8 TB/s; call bytes = the calibrated FETCH_SIZE + WRITE_SIZE bytes of every",
           "kernel of the call (profiles/traffic.json, stored for the bf16 workloads) over the",
           "algorithmic bytes; GEMM = torch's 8192^3 bf16 GEMM on the same box, as a gauge of",
           "the box; cpu = the float64 oracle's TFLOP/s on a bounded sample."]
    for i, d in enumerate(dirs):
        lines = []
        for w in range(1, 6):
            path = os.path.join(d, f"bench_w{w}.log")
            if os.path.exists(path):
                lines.append((w, bench_line(path)))
        out += ["", f"## Box {i + 1} (logs in {d})", "",
                "| W | workload | splits | dtype | value TFLOP/s | ms/step | steps/s | phase kernel "
                "| phase TFLOP/s | frac of MFMA peak | HBM frac | call bytes / algorithmic "
                "| GEMM bf16 TFLOP/s | cpu oracle TFLOP/s |",
                "|" + "---|" * 14]
        for w, ln in lines:
            r, h, c = ln["roofline"], ln["hbm"], ln["config"]
            cb = h.get("call_bytes_over_algorithmic")
            out.append(f"| {w} | {c['workload']} | {c['num_splits']} | {ln['dtype']} | "
                       f"{ln['value']} | {ln['ms_per_step']} | {ln['steps_per_s']} | "
                       f"{r['kernel']} | {r['achieved']} | {r['frac']} | {h['frac']} | "
                       f"{'-' if cb is None else cb} | "
                       f"{ln.get('measured_peaks', {}).get('gemm_bf16_TFLOPs', '-')} | "
                       f"{ln['cpu_baseline']['value']} |")
        out += ["", "Full lines:", ""]
        out += ["    " + json.dumps(ln) for _, ln in lines]
    return "\n".join(out) + "\n"


GREEDY_KERNELS = ("build_ddtree_kernel", "pack_tree_kernel", "tree_accept_kernel")


def greedy_trace(kt_dir: str, bench_log: str, cmd: str) -> str:
    rows = sorted(csv.DictReader(open(os.path.join(kt_dir, "kt_kernel_trace.csv"))),
                  key=lambda r: int(r["Start_Timestamp"]))
    per = defaultdict(list)
    info = {}
    for r in rows:
        name = r["Kernel_Name"]
        key = next((k for k in GREEDY_KERNELS if k in name), None)
        if key is None and "sample_tokens_kernel" in name:
            key = "sample_tokens_kernel " + ("bf16" if "<true" in name else "fp32")
        if key is None:
            continue
        per[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        info[key] = (r["VGPR_Count"], r["Accum_VGPR_Count"], r["SGPR_Count"], r["LDS_Block_Size"],
                     r["Grid_Size_X"], r["Workgroup_Size_X"])
    # bench.py draws flat logits first (1 + 10 launches per dtype), then peaked ones
    for dt in ("fp32", "bf16"):
        k = "sample_tokens_kernel " + dt
        if k in per:
            v = per.pop(k)
            half = len(v) // 2
            per[k + " flat"], per[k + " peaked"] = v[:half], v[half:]
            info[k + " flat"] = info[k + " peaked"] = info.pop(k)
    g = bench_line(bench_log).get("greedy_step", {})
    out = ["# rocprofv3 kernel trace: draft-tree build, tree packing, greedy accept, temperature "
           f"draw ({g.get('batch')} trees, budget {g.get('budget')}, depth {g.get('depth')}, "
           f"workload {g.get('workload')})",
           "",
           "Command (from the repository root, on one MI355X; rocprofv3 run from /tmp with "
           "TMPDIR=/tmp):",
           f"  {cmd}",
           "",
           "bench.py captures 64 launches of each of the first three kernels in one HIP graph and",
           "replays it; the temperature draw (node rows x 163840 tokens, T = 0.8) runs 1 + 10",
           "times each on flat N(0, 2) logits and on peaked ones (12 candidates near +24), fp32",
           "and bf16.",
           "",
           "  kernel | dispatches | avg us | median us | min us | VGPR | AGPR | SGPR | LDS bytes "
           "| grid | block"]
    for k in sorted(per):
        v = sorted(per[k])
        out.append(f"  {k} | {len(v)} | {sum(v) / len(v):.2f} | {v[len(v) // 2]:.2f} | "
                   f"{v[0]:.2f} | " + " | ".join(info[k]))
    out += ["",
            "The same process's bench.py greedy_step line (graph replay or ten launches between "
            "two events, per launch):",
            "  " + json.dumps(g)]
    return "\n".join(out) + "\n"


def main(argv):
    if argv[0] == "trace":
        sys.stdout.write(trace(argv[1], argv[2], int(argv[3]), int(argv[4]), argv[5]))
    elif argv[0] == "traffic":
        print(json.dumps(traffic(argv[1], argv[2], argv[3], int(argv[4]), int(argv[5]), argv[6:]),
                         indent=1))
    elif argv[0] == "traffic-text":
        entries = json.load(open(TRAFFIC_JSON))["entries"]
        entry = next(e for e in entries
                     if e["workload"] == argv[1] and e["num_splits"] == int(argv[2]))
        sys.stdout.write(traffic_text(entry, bench_line(argv[3])))
    elif argv[0] == "counters":
        sys.stdout.write(counters(argv[1], argv[2]))
    elif argv[0] == "bench-table":
        sys.stdout.write(bench_table(argv[1:]))
    elif argv[0] == "greedy-trace":
        sys.stdout.write(greedy_trace(argv[1], argv[2], argv[3]))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv[1:])
