#!/usr/bin/env python3
"""Throughput of the quantized-state decode step on one MI355X.

Default workload: the serving-scale GDN pool (B=512 requests, H=32 heads,
d_k=d_v=128, 31 four-bit heads + 1 FP16 pivot head, fp16 row/column scales,
bf16 q/k/v, four layers).  One step = one token through the four layers = four
stq_decode_step launches, each reading and rewriting every state of its layer.
Inputs are resident in HBM before timing (a ring of 16 pre-generated steps,
shared by the layers: values do not change the cost).

Prints one JSON line: head-updates/s (value), tokens/s, algorithmic HBM GB/s
and its fraction of the 8 TB/s peak for the step kernel (per-launch HIP events
on the launch stream), and the CPU oracle's throughput on a bounded sample of
the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

import synth

METRIC = "quantized-state decode head-updates/s and achieved HBM GB/s (% of peak), B=512"
HBM_PEAK_GBS = 8000.0
RING = 16


def state_bytes(w: synth.Workload, bits: np.ndarray) -> list[int]:
    """Bytes of one head's stored state that a step reads (and writes back):
    code rows plus row and column scales when the head has a quantized row."""
    out = []
    for h in range(w.H):
        wid = bits[h * w.dk:(h + 1) * w.dk] if w.unit == "keyrow" else np.full(w.dk, bits[h])
        codes = int(sum(w.dv * int(b) // 8 for b in wid))
        nq = int((wid < 16).sum())  # quantized rows (not fp16 pivots or fp32 rows)
        scales = (w.dk * (2 if w.row_scale == "f16" else 4) + (2 * w.dv if w.col_scale == "f16" else 0)) if nq else 0
        out.append(codes + scales)
    return out


def io_bytes(w: synth.Workload) -> int:
    """Per head-update: q, k, v in, gate and beta in, o out (fp32)."""
    e = 2 if w.io == "bf16" else 4
    gate = 4 * w.dk if w.gate == "keyvec" else 4
    return e * (2 * w.dk + w.dv) + gate + 4 + 4 * w.dv


def launch_bytes(w: synth.Workload, bits: np.ndarray) -> float:
    """Algorithmic HBM bytes of one launch (B requests, all heads of a layer).

    Every-step mode: each head's stored state is read and written once, plus
    the per-head inputs and output.  Windowed mode (W tokens, K entries): the
    average over one window of what a step must touch once -- base state,
    gate, entries and the n stored deltas read; gate, new delta, decayed keys
    written; at the window end the new base and entries written.
    """
    state = sum(state_bytes(w, bits))
    io = w.H * io_bytes(w) + 4
    if w.window == 1:
        return w.B * (2 * state + io)
    W, K, dk, dv = w.window, w.comps, w.dk, w.dv
    per_head = 0.0
    for n in range(W):
        rd = 4 * dk + 6 * K + 4 + n * 4 * (dk + dv)
        wr = 4 * dk + 4 * (dk + dv) + n * 4 * dk + 4
        per_head += rd + wr
    per_head += 6 * K  # new entries at the window end
    return w.B * (state + state / W + w.H * per_head / W + io)


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_recurrent_stq_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"k_step_{workload}_counters.txt")
    try:
        kv = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w: synth.Workload, units: int, steps: int) -> dict:
    """The oracle, as it stands, on `units` seeded (request, head) states of the
    workload for `steps` steps, one oracle call per state-step, spread over
    host threads (the oracle itself is single-threaded per call)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    bits = synth.unit_bits(w)
    cfg = oracle.Cfg.from_workload(w, bits)
    rng = np.random.default_rng(7)
    ub = rng.integers(0, w.B, units)
    uh = rng.integers(0, w.H, units)
    xs = [synth.step_inputs(w, 0, t, ub, uh) for t in range(steps)]
    slots = [cfg.new_slot() for _ in range(units)]
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    gate_vec = w.gate == "keyvec"

    def run(n):
        for t in range(steps):
            x = xs[t]
            cfg.step_head(slots[n], int(uh[n]), x.q[n], x.k[n], x.v[n],
                          x.a[n] if gate_vec else x.a[n], x.beta[n])

    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(run, range(units)))
    dt = time.perf_counter() - t0
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": units * steps / dt, "unit": "head-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} seeded (request, head) states x {steps} steps of {w.name} layer 0 "
                      f"({units * steps} head-updates, {dt:.2f} s wall on {threads} threads, {cpu})"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="serving_gdn", choices=list(synth.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-units", type=int, default=512)
    ap.add_argument("--cpu-steps", type=int, default=96)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="also run a plain device copy of this many bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decode step needs no collective and this "
              "build measures one GPU's share (see the sharding notes); use --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import linear_attention_recurrent_stq_amd as stq

    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = "cuda"
    layers = []
    for l in range(w.layers):
        bits = synth.unit_bits(w, l)
        L = stq.Layout.from_workload(w, bits)
        pool = stq.Pool(L, w.B)
        layers.append((L, pool, bits))
    ids = torch.from_numpy(np.arange(w.B, dtype=np.int32)[::-1].copy()).to(dev)

    io = torch.bfloat16 if w.io == "bf16" else torch.float32
    qs, ks, vs, as_, bs = [], [], [], [], []
    for t in range(RING):
        x = synth.batch_inputs(w, 0, t)
        if w.io == "bf16":
            cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
            qs.append(cv(x.q_bits)); ks.append(cv(x.k_bits)); vs.append(cv(x.v_bits))
        else:
            qs.append(torch.from_numpy(x.q).to(dev)); ks.append(torch.from_numpy(x.k).to(dev))
            vs.append(torch.from_numpy(x.v).to(dev))
        as_.append(torch.from_numpy(x.a).to(dev)); bs.append(torch.from_numpy(x.beta).to(dev))
    o = torch.empty(w.B, w.H, w.dv, dtype=torch.float32, device=dev)
    if w.init != "zero":
        bb, hh = np.meshgrid(np.arange(w.B), np.arange(w.H), indexing="ij")
        for l, (L, pool, _) in enumerate(layers):
            stq.pack(pool, ids, torch.from_numpy(synth.initial_state(w, l, bb, hh)).to(dev))
    torch.cuda.synchronize()

    def one_step(t, evs=None):
        r = t % RING
        for l, (L, pool, _) in enumerate(layers):
            if evs is not None:
                evs[l][0].record()
            stq.decode_step(pool, ids, qs[r], ks[r], vs[r], as_[r], bs[r], o)
            if evs is not None:
                evs[l][1].record()

    for t in range(args.warmup):
        one_step(t)
    torch.cuda.synchronize()
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    K = args.steps
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(w.layers)] for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for t in range(K):
        one_step(args.warmup + t, ev[t])
        if (t + 1) % 512 == 0:
            print(f"# timed step {t + 1}/{K}", file=sys.stderr, flush=True)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    launch_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])

    head_updates = w.B * w.H * w.layers * K
    value = head_updates / (total_ms * 1e-3)
    per_launch_bytes = np.mean([launch_bytes(w, bits) for (_, _, bits) in layers])
    avg_launch_s = float(launch_ms.mean()) * 1e-3
    achieved = per_launch_bytes / avg_launch_s / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "head-updates/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "d_k": w.dk, "d_v": w.dv, "layers": w.layers,
            "unit_bits": {str(b): int(c) for b, c in zip(*np.unique(layers[0][2], return_counts=True))},
            "scales": f"row {w.row_scale}, column {w.col_scale}", "io": w.io, "window": w.window,
            "comps": w.comps, "parallelism": "single GPU",
        },
        "tokens_per_s": round(w.B * K / (total_ms * 1e-3), 1),
        "hbm_gbs": round(achieved, 1),
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "launch_us": {"mean": round(float(launch_ms.mean()) * 1e3, 2),
                      "p10": round(float(np.percentile(launch_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(launch_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(launch_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(w.name),
                     "kernel": "k_win + k_win_end" if w.window > 1 else "k_step",
                     "bytes_per_launch": int(per_launch_bytes)},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_units, args.cpu_steps)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
