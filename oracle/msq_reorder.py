"""CPU oracle: bi-directional channel reordering from a saliency map.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in oracle/.  The
library never does, and this file imports nothing from it.

The "ScaleBITS" summary page (section Approach) reorders weight channels in
both the row and the column direction so that sensitive weights gather into
block-aligned regions, and (section Limitations) leaves the Q and K
projections out of that local reordering; the "SFMP" abstract reorders rows
and columns to aggregate salient weights.  Neither gives the rule.  Reading
(the plainest one): with a non-negative saliency per weight S[n][k], the row
score is the sum of its row and the column score the sum of its column;
perm_row lists the rows by score descending, perm_col the columns likewise,
ties by index ascending (gather convention: reordered row i is original row
perm_row[i]).  With row reordering off (Q and K projections) perm_row is the
identity.  Scores are summed in fp64 here.

Pins (tests/test_oracle_reorder.py): for a rank-1 saliency a b^T the sorted
orders maximise the block concentration sum over blocks of (saliency mass)^2
among all row and column permutations (rearrangement / majorisation),
checked by brute force on small grids with small blocks; valid permutations;
identical channels keep their index order.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def channel_scores(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row and column sums of the saliency map, fp64."""
    S = np.asarray(S, dtype=np.float64)
    return S.sum(axis=1), S.sum(axis=0)


def order_desc(score: np.ndarray) -> np.ndarray:
    """Indices by score descending, ties by index ascending."""
    idx = np.arange(score.shape[0])
    return np.lexsort((idx, -np.asarray(score, dtype=np.float64))).astype(np.int32)


def reorder_channels(S: np.ndarray, reorder_rows: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """(perm_row, perm_col) for saliency map S [N][K] (module docstring)."""
    r, c = channel_scores(S)
    perm_row = order_desc(r) if reorder_rows else np.arange(S.shape[0], dtype=np.int32)
    return perm_row, order_desc(c)


def block_concentration(S: np.ndarray, perm_row: np.ndarray, perm_col: np.ndarray,
                        br: int = 64, bc: int = 128) -> float:
    """Sum over br x bc blocks of the reordered map of (block saliency mass)^2."""
    Sr = np.asarray(S, dtype=np.float64)[np.ix_(perm_row, perm_col)]
    N, K = Sr.shape
    m = Sr.reshape(N // br, br, K // bc, bc).sum(axis=(1, 3))
    return float((m * m).sum())
