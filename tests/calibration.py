"""Calibration statistics computed with the oracle (test side): the
unquantized fp32 recurrence of each sampled (request, head) state from the
zero state, per-unit gate means and mean squared state entries, accumulated
in float64.  The same definitions as the library's calibrate(); the widths
for allocated workloads in the tests come from these statistics and the
allocation oracle, never from the HIP path."""
from __future__ import annotations

import numpy as np

import oracle
import synth
from oracle import allocator


def oracle_calibration(w: synth.Workload, layer: int, B: int, steps: int, warmup: int | None = None):
    keyrow = w.unit == "keyrow"
    keyvec = w.gate == "keyvec"
    warmup = steps // 2 if warmup is None else warmup
    gsum = np.zeros((w.H, w.dk if keyvec else 1))
    ssum = np.zeros((w.H, w.dk))
    M = [[np.zeros((w.dk, w.dv), np.float32) for _ in range(w.H)] for _ in range(B)]
    n_state = 0
    for t in range(steps):
        x = synth.step_inputs(w, layer, t, np.arange(B)[:, None], np.arange(w.H)[None, :])
        gsum += (x.a.astype(np.float64) if keyvec else x.a.astype(np.float64)[..., None]).sum(axis=0)
        for b in range(B):
            for h in range(w.H):
                oracle.step_f32(M[b][h], x.q[b, h], x.k[b, h], x.v[b, h], x.a[b, h], x.beta[b, h], keyvec)
        if t >= warmup:
            for b in range(B):
                for h in range(w.H):
                    ssum[h] += (M[b][h].astype(np.float64) ** 2).sum(axis=1)
            n_state += 1
    g = gsum / (steps * B)
    m = ssum / (n_state * B * w.dv)
    if keyrow:
        return (np.broadcast_to(g, (w.H, w.dk)).reshape(-1).astype(np.float32),
                m.reshape(-1).astype(np.float32))
    return g.mean(axis=1).astype(np.float32), m.mean(axis=1).astype(np.float32)


def allocated_bits(w: synth.Workload, layer: int = 0, B: int = 8, steps: int = 48, avg_bits: float = 6.0):
    """Widths of an allocated workload from the oracle's calibration and the
    allocation oracle: mean `avg_bits` over non-pivot units, pivot_frac of
    the units (at least one) kept as FP16 pivots."""
    g, m = oracle_calibration(w, layer, B, steps)
    n = g.size
    pivots = max(1, int(round(w.pivot_frac * n))) if w.pivot_frac > 0 else 0
    return np.array(allocator.allocate(g.tolist(), m.tolist(), avg_bits, pivots), np.uint8), g, m


def query_impact(w: synth.Workload, layer: int, B: int, steps: int) -> np.ndarray:
    """Row-impact scores iota_i = E[q_i^2] per (head, key row) from the
    calibration queries (the first B requests, `steps` steps), float32 [H*d_k]:
    an error in row i of the state reaches the output through q_i."""
    acc = np.zeros((w.H, w.dk))
    for t in range(steps):
        x = synth.step_inputs(w, layer, t, np.arange(B)[:, None], np.arange(w.H)[None, :])
        acc += (x.q.astype(np.float64) ** 2).sum(axis=0)
    return (acc / (B * steps)).reshape(-1).astype(np.float32)
