"""Pins of the bit-allocation oracle (oracle/msq_alloc.py) against brute force,
closed forms and a hand-worked instance."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import msq_alloc as A
from block_wise_mixed_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "alloc_worked_example.json")


def _brute(u, budget):
    best = -np.inf
    for lv in itertools.product(range(len(A.LEVELS)), repeat=u.shape[0]):
        bits = [A.LEVELS[l] for l in lv]
        if sum(bits) <= budget:
            best = max(best, float(sum(u[i, l] for i, l in enumerate(lv))))
    return best


@pytest.mark.parametrize("seed", range(6))
def test_dp_matches_brute_force(seed):
    g = np.random.default_rng(seed)
    u = np.cumsum(g.uniform(-1, 3, (4, 6)), axis=1).astype(np.float32)  # any shape, not only concave
    for budget in (0, 1, 3, 7, 12, 20, 32):
        value, bits = A.alloc_optimal(u, budget)
        assert abs(value - _brute(u.astype(np.float64), budget)) < 1e-9
        assert int(bits.astype(int).sum()) <= budget
        assert abs(A.utility(u, bits) - value) < 1e-9


@pytest.mark.parametrize("seed", range(5))
def test_greedy_within_one_step_of_optimum(seed):
    """Concave utilities: classic greedy never beats the optimum and loses at most one
    step's gain (the fractional-knapsack bound)."""
    u = synth.draw_alloc_utility(7, seed)
    gains = np.diff(u.astype(np.float64), axis=1)
    for budget in (2, 5, 9, 14, 21, 30):
        opt, _ = A.alloc_optimal(u, budget)
        got = A.utility(u, A.alloc_greedy(u, budget))
        assert got <= opt + 1e-6
        assert got >= opt - gains.max() - 1e-6


def test_worked_example():
    g = json.load(open(GOLDEN))
    u = np.asarray(g["utility"], dtype=np.float32)
    assert tuple(g["levels"]) == A.LEVELS
    assert A.alloc_greedy(u, g["budget"]).tolist() == g["greedy_bits"]
    bits, iters = A.alloc_batched(u, g["budget"])
    assert bits.tolist() == g["batched_bits"] and iters == g["batched_iterations"]
    assert A.utility(u, bits) == pytest.approx(g["batched_value"])
    assert A.alloc_optimal(u, g["budget"])[0] == pytest.approx(g["optimal_value"])


def test_identical_blocks():
    """Identical blocks: greedy gives floor/ceil of budget / blocks with the extra bit
    on the lowest indices; batched gives bits differing by at most one level."""
    u = np.tile(synth.draw_alloc_utility(1, 3), (10, 1))
    g = A.alloc_greedy(u, 23)
    assert g.tolist() == [3, 3, 3] + [2] * 7
    b, _ = A.alloc_batched(u, 23)
    lv = np.searchsorted(A.LEVELS, b.astype(int))
    assert int(b.astype(int).sum()) == 23 and lv.max() - lv.min() <= 1


@pytest.mark.parametrize("fn", ["greedy", "batched"])
@pytest.mark.parametrize("n,avg", [(200, 0.5), (200, 2.1), (300, 3.9), (50, 8.0)])
def test_budget_and_slack(fn, n, avg):
    """Never over budget; budget left over only when no remaining step fits it."""
    u = synth.draw_alloc_utility(n, 11)
    budget = int(avg * n)
    bits = A.alloc_greedy(u, budget) if fn == "greedy" else A.alloc_batched(u, budget)[0]
    used = int(bits.astype(int).sum())
    assert used <= budget
    left = budget - used
    lv = np.searchsorted(A.LEVELS, bits.astype(int))
    movable = lv < len(A.LEVELS) - 1
    if movable.any():
        nxt = np.asarray(A.LEVELS)[lv[movable] + 1] - bits[movable].astype(int)
        assert left < nxt.min()


def test_greedy_monotone_in_budget():
    """Sensitivities within a factor 10 (every 4 -> 8 step ranks after every unit step):
    more budget never lowers a block's bits under classic greedy."""
    u = synth.draw_alloc_utility(40, 5, sigma=0.5, lo=1.0, hi=10.0)
    prev = A.alloc_greedy(u, 0)
    for budget in range(1, 161, 7):
        cur = A.alloc_greedy(u, budget)
        assert (cur >= prev).all()
        prev = cur


def test_batched_iterations_logarithmic():
    n = 20000
    u = synth.draw_alloc_utility(n, 7)
    bits, iters = A.alloc_batched(u, int(2.1 * n))
    assert int(bits.astype(int).sum()) <= int(2.1 * n)
    assert 10 <= iters <= 40, iters
