"""GPU parity of the bit allocation (msq_allocate_bits) with the oracle's batched
greedy: the same bits for every block and the same iteration count.  Ratios are
formed and compared in fp32 on both sides, so the decisions must agree exactly."""
import json
import os

import numpy as np
import pytest

from oracle import msq_alloc as A
from block_wise_mixed_amd import synth

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def msq():
    import block_wise_mixed_amd as m
    m.load_library()
    assert torch.cuda.is_available()
    return m


def _check(msq, u, budget):
    print(f"alloc n={u.shape[0]} budget={budget}", flush=True)
    bits, iters = msq.allocate_bits(u, budget)
    torch.cuda.synchronize()
    ref, ref_iters = A.alloc_batched(u, budget)
    got = bits.cpu().numpy()
    assert np.array_equal(got, ref), int(np.count_nonzero(got != ref))
    assert iters == ref_iters
    assert int(got.astype(np.int64).sum()) <= budget
    return got, iters


@pytest.mark.parametrize("n,avg,seed", [(1000, 2.1, 1), (5000, 0.7, 2), (20000, 3.3, 3),
                                        (104448, 2.1, 4), (777, 7.9, 5)])
def test_matches_oracle(msq, n, avg, seed):
    """Sizes up to one 70B decoder layer's blocks (104448), ragged counts, budgets from
    below one bit to nearly all-8-bit."""
    _check(msq, synth.draw_alloc_utility(n, seed), int(avg * n))


def test_edge_budgets(msq):
    u = synth.draw_alloc_utility(3000, 9)
    got, iters = _check(msq, u, 0)
    assert (got == 0).all() and iters == 0
    got, _ = _check(msq, u, 8 * 3000)
    assert (got == 8).all()
    got, _ = _check(msq, u, 8 * 3000 + 12345)
    assert (got == 8).all()
    _check(msq, u[:1], 5)


def test_ties_by_block_index(msq):
    """Identical blocks (every ratio tied) and a few distinct values repeated: the order
    falls back to block index on both sides."""
    _check(msq, np.tile(synth.draw_alloc_utility(1, 3), (4099, 1)), 4099 * 2 + 17)
    base = synth.draw_alloc_utility(5, 6)
    _check(msq, base[np.arange(6000) % 5], 6000 * 2 + 3)


def test_worked_example(msq):
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "alloc_worked_example.json")))
    u = np.asarray(g["utility"], dtype=np.float32)
    got, iters = _check(msq, u, g["budget"])
    assert got.tolist() == g["batched_bits"] and iters == g["batched_iterations"]


def test_rejects_non_finite(msq):
    u = synth.draw_alloc_utility(100, 1)
    u[17, 3] = np.nan
    with pytest.raises(msq.MsqError):
        msq.allocate_bits(u, 200)
