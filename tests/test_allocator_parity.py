"""stq_allocate_bits (the library, through the C ABI) against the bit-allocation
oracle: identical widths on seeded statistics, and argument validation.  Host
only: no GPU is involved."""
import ctypes as C

import numpy as np
import pytest

from oracle import allocator as al


@pytest.fixture(scope="module")
def stq():
    import linear_attention_recurrent_stq_amd as stq
    return stq


def _stats(n, seed):
    rng = np.random.default_rng(seed)
    # gates like the workloads' (GDN exp(-softplus(x)/10), KDA 0.8 + 0.2 sigmoid)
    a = np.where(rng.random(n) < 0.5, np.exp(-np.log1p(np.exp(rng.standard_normal(n))) / 10),
                 0.8 + 0.2 / (1 + np.exp(-rng.normal(2, 1, n)))).astype(np.float32)
    m = rng.lognormal(-2.0, 1.5, n).astype(np.float32)
    # a few repeated statistics, so that ties occur
    a[::17] = a[0]
    m[::17] = m[0]
    return a, m


@pytest.mark.parametrize("n,avg,piv", [(1, 4.0, 0), (1, 8.0, 1), (7, 6.0, 1), (32, 6.0, 1),
                                       (32, 4.0, 1), (96, 5.5, 3), (4096, 4.0, 41),
                                       (4096, 6.0, 41), (4096, 7.3, 0)])
def test_library_matches_oracle(stq, n, avg, piv):
    a, m = _stats(n, n + piv)
    got = stq.allocate_bits(a, m, avg, piv)
    want = np.array(al.allocate(a.astype(np.float64).tolist(), m.astype(np.float64).tolist(), avg, piv),
                    np.uint8)
    assert np.array_equal(got, want)


def test_widths_feed_a_layout(stq):
    # KDA per key row: H * d_k units; the result is a valid unit_bits map
    import synth
    w = synth.WORKLOADS["kimi_kda"]
    a, m = _stats(w.H * w.dk, 5)
    bits = stq.allocate_bits(a, m, 4.5, 41)
    L = stq.Layout.from_workload(w, bits)
    assert L.slot_bytes > 0 and set(np.unique(bits)) <= {4, 6, 8, 16}


@pytest.mark.parametrize("case", ["n0", "avg_low", "avg_high", "piv_neg", "piv_big", "gate_neg",
                                  "gate_big", "msq_neg", "msq_inf", "nan_gate", "null"])
def test_invalid_arguments_write_nothing(stq, case):
    a, m = _stats(8, 0)
    n, avg, piv = 8, 6.0, 1
    if case == "n0":
        n = 0
    elif case == "avg_low":
        avg = 3.99
    elif case == "avg_high":
        avg = 8.01
    elif case == "piv_neg":
        piv = -1
    elif case == "piv_big":
        piv = 9
    elif case == "gate_neg":
        a[3] = -0.1
    elif case == "gate_big":
        a[3] = 1.5
    elif case == "msq_neg":
        m[2] = -1.0
    elif case == "msq_inf":
        m[2] = np.inf
    elif case == "nan_gate":
        a[5] = np.nan
    out = np.full(8, 77, np.uint8)
    lib = stq.library()
    ga = None if case == "null" else C.c_void_p(a.ctypes.data)
    st = lib.stq_allocate_bits(n, ga, C.c_void_p(m.ctypes.data), avg, piv, C.c_void_p(out.ctypes.data))
    assert st == stq.STQ_ERR_INVALID
    assert (out == 77).all()
    assert lib.stq_last_error()
