"""CPU oracle: bitwidth allocation per 64x128 block under a memory budget.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in oracle/.  The
library never does, and this file imports nothing from it.

The "ScaleBITS" summary page (sections Approach and Key results) states the
problem: precision is chosen per 64x128 block so as to maximise the model's
quality under a global memory budget, a knapsack over block bitwidths, and
its search is a batched approximation to the classic greedy algorithm (16 to
36 batched iterations where classic greedy needs millions of single steps).
The pages give neither the gain model nor the batching rule.  Readings:

* Each block i has a utility u[i][l] for every level l of LEVELS (given;
  synthetic in the tests), and the cost of level l is LEVELS[l] bits per
  weight (codes only).  Budget: sum over blocks of the chosen bits <= budget.
  A block moves up one level at a time; the step from level l to l + 1 costs
  d = LEVELS[l+1] - LEVELS[l] and gains u[i][l+1] - u[i][l].
* Ratio of a step: r = fp32(u[i][l+1] - u[i][l]) / fp32(d), both operations
  in IEEE fp32 (the precision in which both implementations take their
  decisions).  Order of steps: r descending, then block index ascending.
* classic greedy: from all blocks at level 0, repeatedly take the first step
  in that order whose cost fits the remaining budget R; stop when none fits.
* batched greedy: each iteration orders every block's next step, takes the
  longest prefix whose total cost is at most floor(R / 2), and applies all of
  it at once (a block moves at most one level per iteration); when that
  prefix is empty it takes the first step that fits R, as classic greedy
  would; it stops when nothing fits.  Halving the remaining budget per
  iteration gives about log2(budget) iterations, the pages' 16 to 36.

Pins (tests/test_oracle_alloc.py): the exact dynamic program against brute
force over every assignment of tiny instances; classic greedy never above the
optimum and, for concave utilities, within one step's gain of it; a hand-
worked instance (tests/golden/alloc_worked_example.json); identical blocks
end with bits differing by at most one level, the extra bits on the lowest
indices for classic greedy; budget respected and at most one step of slack;
classic greedy monotone in the budget.  The batching rule itself has no page
to pin it to: parity unpinned for the rule, pinned only in the properties
above.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

LEVELS = (0, 1, 2, 3, 4, 8)


def _steps(u: np.ndarray, lev: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Blocks that can move up, the cost and the fp32 ratio of their next step."""
    L = np.asarray(LEVELS, dtype=np.int64)
    nl = len(LEVELS)
    idx = np.nonzero(lev < nl - 1)[0]
    cur = lev[idx]
    d = L[cur + 1] - L[cur]
    gain = (u[idx, cur + 1].astype(np.float32) - u[idx, cur].astype(np.float32)).astype(np.float32)
    r = (gain / d.astype(np.float32)).astype(np.float32)
    return idx, d, r


def _order(idx: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Positions of the steps sorted by ratio descending, then block index ascending."""
    return np.lexsort((idx, -r))


def alloc_greedy(u: np.ndarray, budget: int) -> np.ndarray:
    """Classic greedy: one step at a time (module docstring).  Returns bits per block."""
    u = np.asarray(u, dtype=np.float32)
    lev = np.zeros(u.shape[0], dtype=np.int64)
    R = int(budget)
    while True:
        idx, d, r = _steps(u, lev)
        took = False
        for p in _order(idx, r):
            if d[p] <= R:
                lev[idx[p]] += 1
                R -= int(d[p])
                took = True
                break
        if not took:
            break
    return np.asarray(LEVELS, dtype=np.uint8)[lev]


def alloc_batched(u: np.ndarray, budget: int) -> Tuple[np.ndarray, int]:
    """Batched greedy (module docstring).  Returns (bits per block, iterations)."""
    u = np.asarray(u, dtype=np.float32)
    lev = np.zeros(u.shape[0], dtype=np.int64)
    R = int(budget)
    iters = 0
    while True:
        idx, d, r = _steps(u, lev)
        if idx.size == 0:
            break
        o = _order(idx, r)
        cum = np.cumsum(d[o])
        p = int(np.searchsorted(cum, R // 2, side="right"))  # longest prefix with cum <= R/2
        if p > 0:
            take = o[:p]
        else:
            fit = np.nonzero(d[o] <= R)[0]
            if fit.size == 0:
                break
            take = o[fit[:1]]
        lev[idx[take]] += 1
        R -= int(d[take].sum())
        iters += 1
    return np.asarray(LEVELS, dtype=np.uint8)[lev], iters


def utility(u: np.ndarray, bits: np.ndarray) -> float:
    """Total utility of an allocation, in fp64."""
    lev = np.searchsorted(np.asarray(LEVELS), np.asarray(bits, dtype=np.int64))
    return float(np.asarray(u, dtype=np.float64)[np.arange(len(lev)), lev].sum())


def alloc_optimal(u: np.ndarray, budget: int) -> Tuple[float, np.ndarray]:
    """Exact knapsack by dynamic programming over (block, bits used), fp64.
    Small budgets only (O(blocks x budget x levels))."""
    u = np.asarray(u, dtype=np.float64)
    n = u.shape[0]
    B = int(budget)
    neg = -np.inf
    best = np.full(B + 1, neg)
    best[0] = 0.0
    choice: List[np.ndarray] = []
    for i in range(n):
        nb = np.full(B + 1, neg)
        ch = np.zeros(B + 1, dtype=np.int64)
        for l, b in enumerate(LEVELS):
            if b > B:
                continue
            cand = np.full(B + 1, neg)
            cand[b:] = best[:B + 1 - b] + u[i, l]
            better = cand > nb
            nb[better] = cand[better]
            ch[better] = l
        best = nb
        choice.append(ch)
    used = int(np.argmax(best))
    value = float(best[used])
    lev = np.zeros(n, dtype=np.int64)
    for i in range(n - 1, -1, -1):
        l = int(choice[i][used])
        lev[i] = l
        used -= LEVELS[l]
    return value, np.asarray(LEVELS, dtype=np.uint8)[lev]
