"""Summaries of rocprofv3 output for the decode kernels (text files under profiles/).

  python -m linear_attention_recurrent_stq_amd.rocprof_summary stats DIR WORKLOAD CMD OUT
      kernel-trace statistics (<DIR>/*_kernel_stats.csv) of the decode kernels
  python -m linear_attention_recurrent_stq_amd.rocprof_summary counters FETCH_DIR WRITE_DIR WORKLOAD COPY_BYTES CMD OUT
      HBM bytes per decode call from a FETCH_SIZE pass and a WRITE_SIZE pass,
      each scaled by what the same counter reads for the plain device copy of
      COPY_BYTES bytes (read COPY_BYTES + write COPY_BYTES) in the same run.

  python -m linear_attention_recurrent_stq_amd.rocprof_summary valu DIR WORKLOAD CMD OUT
      VALU instructions per stq_decode_step call from an SQ_INSTS_VALU /
      SQ_WAVES pass, and VALU issues per state element (x 64 lanes / elements)

CMD is the command line that produced DIR (recorded in the summary).  The
decode kernels are k_step (every-step mode), k_step_lag (lagged scales; the
fit of the next scales, k_fit, is a separate call and not counted) and k_win +
k_win_end (windowed: one stq_decode_step call launches both).
"""
from __future__ import annotations

import csv
import glob
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STEP_KERNELS = ("::k_step<", "::k_step_lag<", "::k_win<", "::k_win_end<")
COPY_KERNEL = "copyBuffer"


def _is_step(name: str) -> bool:
    return any(k in name for k in STEP_KERNELS)


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def stats(d: str, workload: str, cmd: str, out: str) -> None:
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*kernel_stats.csv")))))
    lines = [f"# rocprofv3 kernel-trace statistics, workload {workload}",
             f"# command: {cmd}",
             f"# kernel_source_sha256: {_source_hash(workload)}",
             "kernel | calls | average_us | min_us | max_us | percent"]
    for r in rows:
        lines.append(f"{r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter(d: str, name: str):
    rows = list(csv.DictReader(open(_one(os.path.join(d, "**", "*counter_collection.csv")))))
    per = defaultdict(float)   # dispatch -> value
    kern, grid = {}, {}
    for r in rows:
        if r["Counter_Name"] != name:
            continue
        did = int(r["Dispatch_Id"])
        per[did] += float(r["Counter_Value"])
        kern[did] = r["Kernel_Name"]
        grid[did] = int(r["Grid_Size"])
    step = [per[i] for i in sorted(per) if _is_step(kern[i])]
    step_names = sorted({kern[i] for i in per if _is_step(kern[i])})
    by_kernel = defaultdict(float)
    for i in per:
        if _is_step(kern[i]):
            by_kernel[_short(kern[i])] += per[i]
    # The runtime also issues small copies of its own (argument uploads); the
    # calibration copies are the ones with the largest grid.
    copies = [i for i in per if COPY_KERNEL in kern[i]]
    big = max((grid[i] for i in copies), default=0)
    copy = [per[i] for i in sorted(copies) if grid[i] == big]
    return step, step_names, copy, by_kernel


def _short(name: str) -> str:
    """k_win, k_win_end, k_step, k_step_lag from a demangled kernel name."""
    for k in ("::k_win_end<", "::k_win<", "::k_step_lag<", "::k_step<"):
        if k in name:
            return k[2:-1]
    return name


def _source_hash(workload: str) -> str:
    """Hash of the device sources of the workload's decode kernels."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    return bench.kernel_source_hash(synth.WORKLOADS[workload])


def counters(fetch_dir: str, write_dir: str, workload: str, copy_bytes: int, cmd: str, out: str) -> None:
    sys.path.insert(0, ROOT)
    import bench
    import synth
    w = synth.WORKLOADS[workload]
    f_step, names, f_copy, f_by = _counter(fetch_dir, "FETCH_SIZE")
    w_step, _, w_copy, w_by = _counter(write_dir, "WRITE_SIZE")
    if not f_copy or not w_copy:
        raise SystemExit("the calibration copy kernel is missing from the counter runs")
    kernels_per_call = 2 if w.window > 1 else 1
    calls_f = len(f_step) // kernels_per_call
    calls_w = len(w_step) // kernels_per_call
    fetch_scale = copy_bytes / (sum(f_copy) / len(f_copy) * 1024)
    write_scale = copy_bytes / (sum(w_copy) / len(w_copy) * 1024)
    rd = sum(f_step) / calls_f * 1024 * fetch_scale
    wr = sum(w_step) / calls_w * 1024 * write_scale
    alg = sum(bench.launch_bytes(w, synth.unit_bits(w, l)) for l in range(w.layers)) / w.layers
    lines = [f"# rocprofv3 HBM counters per stq_decode_step call, workload {workload}",
             f"# command: {cmd}",
             f"# scaling: each counter is multiplied by (true bytes / counter bytes) of a plain "
             f"device copy of {copy_bytes} bytes in the same run",
             f"workload: {workload}",
             f"kernels: {', '.join(names)}",
             f"kernel_source_sha256: {_source_hash(workload)}",
             f"calls_measured: {calls_f}",
             f"fetch_scale: {fetch_scale:.4f}",
             f"write_scale: {write_scale:.4f}",
             f"hbm_read_bytes_per_launch: {rd:.0f}",
             f"hbm_write_bytes_per_launch: {wr:.0f}",
             f"hbm_bytes_per_launch: {rd + wr:.0f}",
             f"algorithmic_bytes_per_launch: {alg:.0f}",
             f"traffic_over_algorithmic: {(rd + wr) / alg:.4f}"]
    if len(f_by) > 1:
        # one stq_decode_step call launches several kernels: bytes of each
        for k in sorted(f_by):
            kr = f_by[k] / calls_f * 1024 * fetch_scale
            kw = w_by.get(k, 0.0) / calls_w * 1024 * write_scale
            lines.append(f"{k}_read_bytes_per_call: {kr:.0f}")
            lines.append(f"{k}_write_bytes_per_call: {kw:.0f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def valu(d: str, workload: str, cmd: str, out: str) -> None:
    sys.path.insert(0, ROOT)
    import synth
    w = synth.WORKLOADS[workload]
    insts, names, _, _ = _counter(d, "SQ_INSTS_VALU")
    waves, _, _, _ = _counter(d, "SQ_WAVES")
    if not insts or not waves:
        raise SystemExit("no decode-kernel dispatch in the counter run")
    # one stq_decode_step call launches k_win and k_win_end in the windowed mode
    calls = len(insts) // (2 if w.window > 1 else 1)
    per_launch = sum(insts) / calls
    waves_per_launch = sum(waves) / calls
    elements = w.B * w.H * w.dk * w.dv
    lines = [f"# rocprofv3 VALU instruction counts per stq_decode_step call, workload {workload}",
             f"# command: {cmd}",
             f"workload: {workload}",
             f"kernels: {', '.join(names)}",
             f"kernel_source_sha256: {_source_hash(workload)}",
             f"calls_measured: {calls}",
             f"sq_insts_valu_per_launch: {per_launch:.0f}",
             f"sq_waves_per_launch: {waves_per_launch:.0f}",
             f"valu_insts_per_wave: {per_launch / waves_per_launch:.1f}",
             f"state_elements_per_launch: {elements}",
             f"valu_issues_per_element: {per_launch * 64 / elements:.2f}"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    a = sys.argv[1:]
    if a and a[0] == "stats" and len(a) == 5:
        stats(a[1], a[2], a[3], a[4])
    elif a and a[0] == "counters" and len(a) == 7:
        counters(a[1], a[2], a[3], int(a[4]), a[5], a[6])
    elif a and a[0] == "valu" and len(a) == 5:
        valu(a[1], a[2], a[3], a[4])
    else:
        raise SystemExit(__doc__)
