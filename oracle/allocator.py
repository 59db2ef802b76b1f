"""Lifetime-aware bit allocation, written plainly (CPU oracle).

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the product
package.  Pure Python on float64; every value a decision depends on is
computed with the same operations, in the same order, as stated below.

What it follows (STEPQuant essay, temporal-axis paragraphs and the
Proposition 1 discussion): an error component that the update does not remove
fades only by the gate, so an error stored in a unit with mean gate a lives
for about sum_t a^t = 1 / (1 - a) steps; within a fixed average width, bits go
to the units whose error is large and long-lived, and a few of the riskiest
units are kept as FP16 pivots.  The pages give no formula; this is the
reading used here:

  lifetime      l_u = 1 / (1 - min(a_u, 1 - 2^-20))        (a_u: mean gate)
  weight        s_u = l_u * m_u                              (m_u: mean squared entry)
  risk at b     r_u(b) = s_u * 4^-b   (a uniform step's squared error scales as 4^-b)
  pivots        the P units of largest s_u (ties: lower index) become width 16
  widths        every other unit starts at 4; the budget is floor(avg * N')
                bits over the N' = N - P other units; while 2 more bits fit,
                the unit with the largest gain r_u(b) - r_u(b + 2) (b < 8;
                ties: lower index) moves to b + 2.
  gain          g_u(b) = s_u * (15 * 2^-(2b + 4))   (= 4^-b - 4^-(b+2), exact)

Each unit's gains shrink 16-fold per step, so the greedy choice minimises the
total risk sum_u r_u(b_u) over the assignments within the budget.
"""
from __future__ import annotations

import math

WIDTHS = (4, 6, 8)
PIVOT = 16
GATE_CAP = 1.0 - 2.0 ** -20


def lifetime(a: float) -> float:
    return 1.0 / (1.0 - min(float(a), GATE_CAP))


def weight(a: float, m: float) -> float:
    return lifetime(a) * float(m)


def gain(s: float, b: int) -> float:
    """r(b) - r(b + 2) for weight s: s * 15 * 2^-(2b+4) (the factor is exact)."""
    return s * (15.0 * math.ldexp(1.0, -(2 * b + 4)))


def risk(s: float, b: int) -> float:
    return s * math.ldexp(1.0, -2 * b)


def allocate(gate_mean, state_msq, avg_bits: float, n_pivots: int) -> list[int]:
    """Widths per unit (4/6/8, or 16 for a pivot)."""
    n = len(gate_mean)
    assert len(state_msq) == n and 0 <= n_pivots <= n and 4.0 <= avg_bits <= 8.0
    s = [weight(gate_mean[u], state_msq[u]) for u in range(n)]
    # pivots: largest weight first, lower index first among equals
    order = sorted(range(n), key=lambda u: (-s[u], u))
    bits = [4] * n
    for u in order[:n_pivots]:
        bits[u] = PIVOT
    rest = [u for u in range(n) if bits[u] != PIVOT]
    budget = math.floor(avg_bits * len(rest))
    used = 4 * len(rest)
    # plain greedy: scan every unit for the largest gain of its next 2 bits
    # (a unit at 8 bits, or a pivot, offers none); the first maximum in index
    # order wins ties
    while used + 2 <= budget:
        best, best_gain = -1, -1.0
        for u in rest:
            if bits[u] < 8:
                gu = gain(s[u], bits[u])
                if gu > best_gain:
                    best, best_gain = u, gu
        if best < 0:
            break
        bits[best] += 2
        used += 2
    return bits
