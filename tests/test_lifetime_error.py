"""A synthetic Fig. 1(b) of the STEPQuant essay (temporal-axis paragraphs:
cells that hold memory longer accumulate more error when stored coarsely),
measured with the oracle, and the two premises of the lifetime-aware bit
allocation checked against it: the error a unit accumulates grows with its
lifetime 1/(1 - a), and two more bits divide it by about 4^2 = 16.

KDA state, d_k = d_v = 32, key rows in four classes of fixed gate a = 0.5,
0.8, 0.95, 0.99 (lifetimes 2, 5, 20, 100 steps), every row stored at 4, 6 or
8 bits with dual-axis scales refitted each step; unit-norm random keys and
queries, N(0,1) values, write strength U(0.2, 0.8); 300 steps from the zero
state, six seeded runs.  Error = stored state minus the exact (fp64)
recurrence on the same inputs, mean square per row over steps 150..299.
"""
import numpy as np

GATES = (0.5, 0.8, 0.95, 0.99)


def _measure(ora, width, dk=32, dv=32, steps=300, runs=6, seed=0):
    rng = np.random.default_rng(seed + width)
    gates = np.repeat(np.array(GATES), dk // len(GATES)).astype(np.float32)
    bits = np.full(dk, width, np.uint8)
    cfg = ora.Cfg(1, dk, dv, True, True, True, True, 1, 0, bits)
    err = np.zeros(dk)
    mag = np.zeros(dk)
    for _ in range(runs):
        slot = cfg.new_slot()
        M = np.zeros((dk, dv))
        n = 0
        for t in range(steps):
            k = rng.standard_normal(dk); k /= np.linalg.norm(k)
            q = rng.standard_normal(dk); q /= np.linalg.norm(q)
            v = rng.standard_normal(dv)
            b = rng.uniform(0.2, 0.8)
            k, q, v = (x.astype(np.float32) for x in (k, q, v))
            cfg.step_head(slot, 0, q, k, v, gates, b)
            ora.step_f64(M, q, k, v, gates, float(np.float32(b)), True)
            if t >= steps // 2:
                E = cfg.unpack_head(slot, 0) - M
                err += (E ** 2).mean(axis=1)
                mag += (M ** 2).mean(axis=1)
                n += 1
    k4 = len(GATES)
    return (err / (n * runs)).reshape(k4, -1).mean(axis=1), (mag / (n * runs)).reshape(k4, -1).mean(axis=1)


def test_error_grows_with_lifetime_and_falls_16x_per_two_bits(ora):
    res = {w: _measure(ora, w) for w in (4, 6, 8)}
    print("\nwidth | " + " | ".join(f"MSE at lifetime {1 / (1 - a):.0f}" for a in GATES))
    for w, (e, m) in res.items():
        print(f"{w} | " + " | ".join(f"{x:.3g} (rel {x / y:.3g})" for x, y in zip(e, m)))
    for w, (e, m) in res.items():
        # longer-lived rows accumulate more error; relative to their size too,
        # where it levels off between the two longest lifetimes
        assert np.all(np.diff(e) > 0), (w, e)
        rel = e / m
        assert rel[1] > rel[0] and rel[2] > rel[1] and min(rel[2], rel[3]) > 2 * rel[0], (w, rel)
    for lo, hi in ((4, 6), (6, 8)):
        ratio = res[lo][0] / res[hi][0]
        assert np.all((ratio > 8) & (ratio < 32)), (lo, hi, ratio)
