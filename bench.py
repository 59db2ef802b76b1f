#!/usr/bin/env python3
"""Throughput of the quantized-state decode step on one MI355X.

Default workload: the serving-scale GDN pool (B=512 requests, H=32 heads,
d_k=d_v=128, 31 four-bit heads + 1 FP16 pivot head, fp16 row/column scales,
bf16 q/k/v, four layers).  One step = one token through the four layers = four
stq_decode_step launches, each reading and rewriting every state of its layer.
Inputs are resident in HBM before timing (a ring of 16 pre-generated steps,
shared by the layers: values do not change the cost).

Protocol: W warm-up steps, continued until at least --warmup-seconds of
warm-up have run (clocks and caches settle; the JSON records how many warm-up
steps ran), then exactly K timed steps between two HIP events on the launch
stream, with a device synchronization on both sides and no other event inside.
A second, untimed pass then records events around each launch to give the
launch-time distribution.

Prints one JSON line: head-updates/s (value), tokens/s, algorithmic HBM GB/s
and its fraction of the 8 TB/s peak for the step kernel (algorithmic bytes per
launch over the timed region's time per launch), and the CPU oracle's
throughput on a bounded sample of the same workload (cpu_baseline, on all
usable host threads up to 16 and on one thread).
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
        if nq and getattr(w, "scale_fit", "step") == "lagged":
            # next scales (read by the step) and statistics (written by it)
            scales += scales + 4 * w.dk + (4 * w.dv if w.col_scale == "f16" else 0)
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


INIT_REQUESTS = 32  # requests whose outlier initial states are drawn (then repeated)

# the sources each decode kernel is compiled from (host-only files excluded):
# the every-step kernels and the windowed ones share only the device headers
STEP_SOURCES = ("stq_device.h", "stq_internal.h", "stq_kernels.hip")
WINDOW_SOURCES = ("stq_device.h", "stq_internal.h", "stq_window.hip")


def kernel_source_hash(w: synth.Workload | None = None) -> str:
    """Hash of the device sources of the workload's decode kernels (every
    device source without a workload)."""
    import hashlib
    files = (WINDOW_SOURCES if w.window > 1 else STEP_SOURCES) if w is not None \
        else tuple(sorted(set(STEP_SOURCES + WINDOW_SOURCES)))
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_recurrent_stq_amd", "csrc")
    for f in sorted(files):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def step_kernel(w: synth.Workload) -> str:
    """Name of the kernel a stq_decode_step call of this workload spends its time in."""
    if w.window > 1:
        return "k_win"
    return "k_step_lag" if w.scale_fit == "lagged" else "k_step"


def counter_traffic(w: synth.Workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{step_kernel(w)}_{w.name}_counters.txt")
    try:
        kv = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("kernel_source_sha256") != kernel_source_hash(w):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _oracle_rate(w: synth.Workload, bits: np.ndarray, units: int, steps: int, threads: int, seed: int,
                 row_impact=None):
    """The oracle, as it stands, on `units` seeded (request, head) states of the
    workload for `steps` steps, one oracle call per state-step, over `threads`
    host threads (the oracle itself is single-threaded per call).  Returns
    (head-updates/s, seconds)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    cfg = oracle.Cfg.from_workload(w, bits, row_impact=row_impact)
    rng = np.random.default_rng(seed)
    ub = rng.integers(0, w.B, units)
    uh = rng.integers(0, w.H, units)
    xs = [synth.step_inputs(w, 0, t, ub, uh) for t in range(steps)]
    slots = [cfg.new_slot() for _ in range(units)]

    def run(n):
        for t in range(steps):
            x = xs[t]
            cfg.step_head(slots[n], int(uh[n]), x.q[n], x.k[n], x.v[n], x.a[n], x.beta[n])

    t0 = time.perf_counter()
    if threads == 1:
        for n in range(units):
            run(n)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, range(units)))
    dt = time.perf_counter() - t0
    return units * steps / dt, dt


def cpu_baseline(w: synth.Workload, bits: np.ndarray, units: int, steps: int, row_impact=None) -> dict:
    """The oracle on this host: all usable threads (at most 16) over disjoint
    states, and one thread on a smaller sample (head-updates/s per core)."""
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    rate, dt = _oracle_rate(w, bits, units, steps, threads, 7, row_impact)
    u1, s1 = 64, 64
    rate1, dt1 = _oracle_rate(w, bits, u1, s1, 1, 8, row_impact)
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(rate, 1), "unit": "head-updates/s", "cores": threads, "kind": "oracle",
            "sample": f"{units} seeded (request, head) states x {steps} steps of {w.name} layer 0 "
                      f"({units * steps} head-updates, {dt:.2f} s wall on {threads} threads, {cpu})",
            "single_thread": {"value": round(rate1, 1), "unit": "head-updates/s", "cores": 1,
                              "sample": f"{u1} states x {s1} steps ({u1 * s1} head-updates, "
                                        f"{dt1:.2f} s on one thread)"}}


CAL_REQUESTS, CAL_STEPS, CAL_AVG_BITS = 32, 64, 6.0


def allocated_widths(stq, torch, w: synth.Workload, layer: int) -> np.ndarray:
    """Widths of an allocated workload through the product path: the library's
    calibration pass (fp32 units) over the first CAL_REQUESTS requests for
    CAL_STEPS steps, then stq_allocate_bits (mean CAL_AVG_BITS bits over the
    non-pivot units, pivot_frac of the units as FP16 pivots)."""
    B = min(CAL_REQUESTS, w.B)

    def inputs(t):
        x = synth.step_inputs(w, layer, t, np.arange(B)[:, None], np.arange(w.H)[None, :])
        if w.io == "bf16":
            cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
            q, k, v = cv(x.q_bits), cv(x.k_bits), cv(x.v_bits)
        else:
            q, k, v = (torch.from_numpy(y).cuda() for y in (x.q, x.k, x.v))
        return q, k, v, torch.from_numpy(x.a).cuda(), torch.from_numpy(x.beta).cuda()

    g, m = stq.calibrate(w.H, w.dk, w.dv, B=B, steps=CAL_STEPS, inputs=inputs,
                         unit=stq.UNIT_KEYROW if w.unit == "keyrow" else stq.UNIT_HEAD,
                         gate=stq.GATE_KEYVEC if w.gate == "keyvec" else stq.GATE_SCALAR,
                         io_dtype=stq.BF16 if w.io == "bf16" else stq.F32)
    pivots = max(1, int(round(w.pivot_frac * g.size))) if w.pivot_frac > 0 else 0
    return stq.allocate_bits(g, m, CAL_AVG_BITS, pivots)


def query_impact(w: synth.Workload, layer: int) -> np.ndarray:
    """Row-impact scores E[q_i^2] per (head, key row) from the calibration
    queries (the first CAL_REQUESTS requests over CAL_STEPS steps)."""
    B = min(CAL_REQUESTS, w.B)
    acc = np.zeros((w.H, w.dk))
    for t in range(CAL_STEPS):
        x = synth.step_inputs(w, layer, t, np.arange(B)[:, None], np.arange(w.H)[None, :])
        acc += (x.q.astype(np.float64) ** 2).sum(axis=0)
    return (acc / (B * CAL_STEPS)).reshape(-1).astype(np.float32)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep warming up (whole steps) until this much time has passed")
    ap.add_argument("--launch-pass", type=int, default=64,
                    help="steps of the untimed pass with events around each launch")
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
    layers, impacts = [], []
    for l in range(w.layers):
        bits = allocated_widths(stq, torch, w, l) if w.bits == "allocated" else synth.unit_bits(w, l)
        impact = query_impact(w, l) if getattr(w, "impact", "none") == "queries" else None
        L = stq.Layout.from_workload(w, bits, row_impact=impact)
        pool = stq.Pool(L, w.B)
        layers.append((L, pool, bits))
        impacts.append(impact)
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
        # seeded outlier states of the first INIT_REQUESTS requests, repeated
        # over the batch: drawing every state of a large pool on the host
        # takes minutes, and the values do not change the cost of a step
        n0 = min(w.B, INIT_REQUESTS)
        bb, hh = np.meshgrid(np.arange(n0), np.arange(w.H), indexing="ij")
        for l, (L, pool, _) in enumerate(layers):
            m0 = torch.from_numpy(synth.initial_state(w, l, bb, hh)).to(dev)
            reps = (w.B + n0 - 1) // n0
            stq.pack(pool, ids, m0.repeat(reps, 1, 1, 1)[: w.B].contiguous())
            del m0
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    # lagged scales: each layer's scale fit runs on a second stream (default
    # priority), after that layer's decode step and before its next one
    lagged = getattr(w, "scale_fit", "step") == "lagged"
    side = torch.cuda.Stream() if lagged else None
    dec_done = [torch.cuda.Event() for _ in layers]
    fit_done = [None for _ in layers]

    def one_step(t, evs=None):
        r = t % RING
        for l, (L, pool, _) in enumerate(layers):
            if fit_done[l] is not None:
                stream.wait_event(fit_done[l])
            if evs is not None:
                evs[l][0].record(stream)
            stq.decode_step(pool, ids, qs[r], ks[r], vs[r], as_[r], bs[r], o, stream=stream)
            if evs is not None:
                evs[l][1].record(stream)
            if lagged:
                dec_done[l].record(stream)
                side.wait_event(dec_done[l])
                stq.fit_scales(pool, ids, stream=side)
                if fit_done[l] is None:
                    fit_done[l] = torch.cuda.Event()
                fit_done[l].record(side)

    # warm-up: W steps, then whole steps until the time budget has passed
    t0 = time.perf_counter()
    nwarm = 0
    while nwarm < args.warmup or time.perf_counter() - t0 < args.warmup_seconds:
        one_step(nwarm)
        nwarm += 1
        if nwarm % 64 == 0 or nwarm == args.warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t0
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for t in range(K):
        one_step(nwarm + t)
        if (t + 1) % 512 == 0:
            print(f"# timed step {t + 1}/{K}", file=sys.stderr, flush=True)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)

    # untimed pass: events around every launch (the kernel-time distribution)
    NP = max(1, args.launch_pass)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(w.layers)] for _ in range(NP)]
    for t in range(NP):
        one_step(nwarm + K + t, ev[t])
    torch.cuda.synchronize()
    launch_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])

    head_updates = w.B * w.H * w.layers * K
    value = head_updates / (total_ms * 1e-3)
    per_launch_bytes = np.mean([launch_bytes(w, bits) for (_, _, bits) in layers])
    avg_launch_s = total_ms * 1e-3 / (K * w.layers)
    achieved = per_launch_bytes / avg_launch_s / 1e9
    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "head-updates/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_run": {"steps": nwarm, "seconds": round(warm_s, 3)},
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
            "scale_fit": getattr(w, "scale_fit", "step") + (" (fit on a second stream)" if lagged else ""),
            "row_impact": ("E[q_i^2] over %d requests x %d calibration steps" % (CAL_REQUESTS, CAL_STEPS)
                           if getattr(w, "impact", "none") == "queries" else None),
            "widths": ("calibrated: fp32-unit recurrence over %d requests x %d steps, then "
                       "stq_allocate_bits at mean %.0f bits" % (CAL_REQUESTS, CAL_STEPS, CAL_AVG_BITS)
                       if w.bits == "allocated" else w.bits),
        },
        "tokens_per_s": round(w.B * K / (total_ms * 1e-3), 1),
        "hbm_gbs": round(achieved, 1),
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "launch_us": {"timed_region_mean": round(avg_launch_s * 1e6, 2),
                      "events_pass_steps": NP,
                      "mean": round(float(launch_ms.mean()) * 1e3, 2),
                      "p10": round(float(np.percentile(launch_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(launch_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(launch_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(w),
                     "kernel": "k_win + k_win_end" if w.window > 1 else step_kernel(w),
                     "bytes_per_launch": int(per_launch_bytes)},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, layers[0][2], args.cpu_units, args.cpu_steps, impacts[0])
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
