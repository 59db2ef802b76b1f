"""The bit-allocation oracle pinned to facts outside it: budget extremes, the
exact bit count, brute-force optimality on tiny inputs, pivot choice,
monotonicity, tie order and the lifetime of a geometric decay."""
import itertools
import math

import numpy as np
import pytest

from oracle import allocator as al


def _rand(n, seed):
    rng = np.random.default_rng(seed)
    a = rng.uniform(0.0, 0.999, n)
    m = rng.lognormal(0.0, 2.0, n)
    return a.tolist(), m.tolist()


def test_lifetime_is_the_sum_of_the_decay():
    # sum_t a^t = 1 / (1 - a): 1 for a = 0, 2 for a = 0.5, 10 for a = 0.9 (to rounding)
    assert al.lifetime(0.0) == 1.0
    assert al.lifetime(0.5) == 2.0
    assert abs(al.lifetime(0.9) - sum(0.9 ** t for t in range(2000))) < 1e-9
    # a gate of 1 never forgets: capped at 2^20 steps
    assert al.lifetime(1.0) == 2.0 ** 20


@pytest.mark.parametrize("pivots", [0, 3])
def test_budget_extremes(pivots):
    a, m = _rand(40, 1)
    b4 = al.allocate(a, m, 4.0, pivots)
    b8 = al.allocate(a, m, 8.0, pivots)
    assert sorted(set(x for x in b4 if x != 16)) == [4]
    assert sorted(set(x for x in b8 if x != 16)) == [8]
    assert b4.count(16) == b8.count(16) == pivots


@pytest.mark.parametrize("avg", [4.0, 4.3, 5.0, 5.99, 6.0, 7.25, 8.0])
def test_bit_count_is_the_budget(avg):
    a, m = _rand(37, 2)
    bits = al.allocate(a, m, avg, 2)
    rest = [b for b in bits if b != 16]
    total = math.floor(avg * len(rest))
    # every 2-bit step that fits is taken: the sum is the budget, or one below it
    assert total - 1 <= sum(rest) <= total
    assert all(b in (4, 6, 8) for b in rest)


@pytest.mark.parametrize("seed", range(12))
def test_greedy_is_optimal_by_brute_force(seed):
    n = 2 + seed % 4
    a, m = _rand(n, 100 + seed)
    avg = [4.5, 5.0, 6.0, 6.5, 7.0, 7.6][seed % 6]
    bits = al.allocate(a, m, avg, 0)
    s = [al.weight(a[u], m[u]) for u in range(n)]
    budget = math.floor(avg * n)
    best = min(sum(al.risk(s[u], c[u]) for u in range(n))
               for c in itertools.product((4, 6, 8), repeat=n) if sum(c) <= budget)
    got = sum(al.risk(s[u], bits[u]) for u in range(n))
    assert got <= best * (1 + 1e-12)


def test_pivots_are_the_largest_weights():
    a, m = _rand(50, 3)
    bits = al.allocate(a, m, 5.0, 4)
    s = np.array([al.weight(a[u], m[u]) for u in range(50)])
    piv = sorted(u for u in range(50) if bits[u] == 16)
    assert piv == sorted(np.argsort(-s, kind="stable")[:4].tolist())


def test_more_weight_never_gets_fewer_bits():
    a, m = _rand(64, 4)
    bits = al.allocate(a, m, 6.0, 0)
    s = [al.weight(a[u], m[u]) for u in range(64)]
    for u in range(64):
        for v in range(64):
            if s[u] > s[v]:
                assert bits[u] >= bits[v]


def test_longer_lifetime_gets_more_bits():
    # same magnitude, gates 0.1 / 0.9 / 0.99: one upgrade each goes to the
    # longest-lived first (budget for two upgrades of three units)
    bits = al.allocate([0.1, 0.9, 0.99], [1.0, 1.0, 1.0], 16 / 3, 0)
    assert bits == [4, 6, 6]
    bits = al.allocate([0.1, 0.9, 0.99], [1.0, 1.0, 1.0], 14 / 3, 0)
    assert bits == [4, 4, 6]


def test_ties_go_to_the_lower_index():
    bits = al.allocate([0.5] * 3, [1.0] * 3, 14 / 3, 0)
    assert bits == [6, 4, 4]
    bits = al.allocate([0.5] * 3, [1.0] * 3, 4.0, 1)
    assert bits == [16, 4, 4]
