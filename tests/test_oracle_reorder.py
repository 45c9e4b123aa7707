"""Pins of the channel-reordering oracle (oracle/msq_reorder.py)."""
import itertools

import numpy as np
import pytest

from oracle import msq_reorder as R
from block_wise_mixed_amd import synth


@pytest.mark.parametrize("seed", range(4))
def test_rank1_sorted_order_maximises_concentration(seed):
    """Rank-1 saliency a b^T: the sorted row and column orders reach the largest block
    concentration over every pair of permutations (brute force, 4x6 map, 2x3 blocks)."""
    g = np.random.default_rng(seed)
    a, b = g.uniform(0.1, 5, 4), g.uniform(0.1, 5, 6)
    S = np.outer(a, b)
    pr, pc = R.reorder_channels(S)
    got = R.block_concentration(S, pr, pc, 2, 3)
    best = max(R.block_concentration(S, np.array(p), np.array(q), 2, 3)
               for p in itertools.permutations(range(4)) for q in itertools.permutations(range(6)))
    assert got == pytest.approx(best, rel=1e-12)


def test_valid_permutations_and_sorted_scores():
    S = synth.draw_saliency(192, 384, 3)
    pr, pc = R.reorder_channels(S)
    assert sorted(pr.tolist()) == list(range(192)) and sorted(pc.tolist()) == list(range(384))
    r, c = R.channel_scores(S)
    assert (np.diff(r[pr]) <= 0).all() and (np.diff(c[pc]) <= 0).all()
    # concentration never below the identity order for this activation-aware map
    ident = (np.arange(192), np.arange(384))
    assert R.block_concentration(S, pr, pc) >= R.block_concentration(S, *ident)


def test_ties_and_rows_off():
    S = np.ones((128, 256), dtype=np.float32)
    S[5] *= 2
    pr, pc = R.reorder_channels(S)
    assert pr[0] == 5 and pr[1:].tolist() == [i for i in range(128) if i != 5]
    assert pc.tolist() == list(range(256))
    pr2, pc2 = R.reorder_channels(S, reorder_rows=False)
    assert pr2.tolist() == list(range(128)) and pc2.tolist() == pc.tolist()
