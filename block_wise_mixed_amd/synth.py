"""Seeded synthetic workloads: weight matrices, bit maps, permutations, activations.

This module only draws inputs.  It holds none of the quantizer's or the
matmul's arithmetic, so the CPU oracle and the HIP path can both be fed from
it without sharing any of the method.  Everything is numpy on the CPU and is
reproducible from seed 0.

Workloads mirror the linear-layer shapes the pages evaluate on (Llama-3-8B and
Llama-3-70B, "ScaleBITS" summary page, sections Key results and Experimental
setup) with random weights in place of trained ones:

* W ~ N(0, 0.02) in fp32 (0.02 is the standard deviation), a set of outlier
  input columns (1% of K, chosen uniformly without replacement in the original
  column order, 4 columns for the 256x512 smoke matrix) multiplied by 10 in
  fp32, then rounded to bf16 (round to nearest even).
* Block bitwidths drawn i.i.d. per 64x128 block from a stated distribution
  over {0,1,2,3,4,8}; the realized mean is whatever the draw gives.
* Uniform random row and column permutations.
* x ~ N(0, 1) rounded to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

import numpy as np

BLOCK_ROWS = 64
BLOCK_COLS = 128

# Bit distributions (probability per block).  Names say what they are.
DIST_SMOKE = {0: 0.05, 1: 0.10, 2: 0.55, 3: 0.15, 4: 0.10, 8: 0.05}
DIST_LABEL_2P1 = {0: 0.05, 1: 0.10, 2: 0.60, 3: 0.15, 4: 0.08, 8: 0.02}
DIST_LABEL_3P0 = {2: 0.30, 3: 0.45, 4: 0.20, 8: 0.05}
# Only "about 2.5 bits over {1,2,3,4,8}" is given for the prefill workload;
# this distribution has mean exactly 2.50.
DIST_LABEL_2P5 = {1: 0.15, 2: 0.45, 3: 0.27, 4: 0.10, 8: 0.03}


@dataclass(frozen=True)
class Matrix:
    name: str
    N: int  # out features
    K: int  # in features


@dataclass(frozen=True)
class Workload:
    index: int          # stream index of this workload under seed 0
    name: str
    matrices: Tuple[Matrix, ...]
    dist: Dict[int, float]
    ms: Tuple[int, ...]
    outlier_frac: float = 0.01
    outlier_count: int = -1   # >= 0 overrides outlier_frac


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload(0, "linear-256x512", (Matrix("lin", 256, 512),), DIST_SMOKE, (1, 4),
                 outlier_count=4),
        Workload(1, "llama3-8b-q_proj", (Matrix("q_proj", 4096, 4096),), DIST_LABEL_2P1, (1,)),
        Workload(2, "llama3-8b-mlp",
                 (Matrix("gate_proj", 14336, 4096), Matrix("up_proj", 14336, 4096),
                  Matrix("down_proj", 4096, 14336)),
                 DIST_LABEL_3P0, (1, 8, 16, 64)),
        Workload(3, "llama3-8b-down_proj-prefill", (Matrix("down_proj", 4096, 14336),),
                 DIST_LABEL_2P5, (512, 2048, 8192)),
        Workload(4, "llama3-70b-layer",
                 (Matrix("q_proj", 8192, 8192), Matrix("k_proj", 1024, 8192),
                  Matrix("v_proj", 1024, 8192), Matrix("o_proj", 8192, 8192),
                  Matrix("gate_proj", 28672, 8192), Matrix("up_proj", 28672, 8192),
                  Matrix("down_proj", 8192, 28672)),
                 DIST_LABEL_2P1, (1, 16, 2048)),
    )
}

# Roles of the independent random streams of one matrix.
_ROLE_W, _ROLE_OUTLIER, _ROLE_BITS, _ROLE_PROW, _ROLE_PCOL, _ROLE_X = range(6)


def rng(workload_index: int, matrix_index: int, role: int, extra: int = 0) -> np.random.Generator:
    """Independent PCG64 stream for (workload, matrix, role, extra), all under seed 0."""
    ss = np.random.SeedSequence(0, spawn_key=(workload_index, matrix_index, role, extra))
    return np.random.default_rng(ss)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_weight(N: int, K: int, n_outliers: int, g_w: np.random.Generator,
                g_out: np.random.Generator, std: float = 0.02) -> np.ndarray:
    """W ~ N(0, std) with n_outliers input columns scaled by 10; bf16 bit patterns [N][K]."""
    w = g_w.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    if n_outliers > 0:
        cols = g_out.choice(K, size=n_outliers, replace=False)
        w[:, cols] *= np.float32(10.0)
    return f32_to_bf16_bits(w)


def draw_bits(N: int, K: int, dist: Dict[int, float], g: np.random.Generator) -> np.ndarray:
    values = np.array(sorted(dist), dtype=np.uint8)
    probs = np.array([dist[int(v)] for v in values], dtype=np.float64)
    probs = probs / probs.sum()
    return g.choice(values, size=(N // BLOCK_ROWS, K // BLOCK_COLS), p=probs).astype(np.uint8)


def draw_perm(n: int, g: np.random.Generator) -> np.ndarray:
    return g.permutation(n).astype(np.int32)


def draw_x(M: int, K: int, g: np.random.Generator) -> np.ndarray:
    return f32_to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))


@dataclass
class MatrixInputs:
    name: str
    N: int
    K: int
    W: np.ndarray          # uint16 bf16 bits [N][K], original order
    bits: np.ndarray       # uint8 [N/64][K/128]
    perm_row: np.ndarray   # int32 [N]
    perm_col: np.ndarray   # int32 [K]
    workload_index: int = 0
    matrix_index: int = 0

    def x(self, M: int) -> np.ndarray:
        """Activations for batch size M (bf16 bits [M][K]); one stream per M."""
        return draw_x(M, self.K, rng(self.workload_index, self.matrix_index, _ROLE_X, M))

    @property
    def mean_bits(self) -> float:
        return float(self.bits.astype(np.float64).mean())


def outlier_count(w: Workload, K: int) -> int:
    return w.outlier_count if w.outlier_count >= 0 else int(round(w.outlier_frac * K))


def matrix_inputs(workload: str, matrix: str | int) -> MatrixInputs:
    """Seeded inputs of one matrix of a named workload."""
    w = WORKLOADS[workload]
    if isinstance(matrix, str):
        mi = [m.name for m in w.matrices].index(matrix)
    else:
        mi = int(matrix)
    m = w.matrices[mi]
    W = draw_weight(m.N, m.K, outlier_count(w, m.K), rng(w.index, mi, _ROLE_W),
                    rng(w.index, mi, _ROLE_OUTLIER))
    bits = draw_bits(m.N, m.K, w.dist, rng(w.index, mi, _ROLE_BITS))
    prow = draw_perm(m.N, rng(w.index, mi, _ROLE_PROW))
    pcol = draw_perm(m.K, rng(w.index, mi, _ROLE_PCOL))
    return MatrixInputs(m.name, m.N, m.K, W, bits, prow, pcol, w.index, mi)


def random_case(N: int, K: int, seed: int, dist: Dict[int, float] | None = None,
                n_outliers: int | None = None, std: float = 0.02) -> MatrixInputs:
    """A free-standing case of any shape (tests): stream index 100 + seed."""
    dist = DIST_SMOKE if dist is None else dist
    n_out = max(1, K // 100) if n_outliers is None else n_outliers
    idx = 100 + seed
    W = draw_weight(N, K, n_out, rng(idx, 0, _ROLE_W), rng(idx, 0, _ROLE_OUTLIER), std)
    bits = draw_bits(N, K, dist, rng(idx, 0, _ROLE_BITS))
    prow = draw_perm(N, rng(idx, 0, _ROLE_PROW))
    pcol = draw_perm(K, rng(idx, 0, _ROLE_PCOL))
    return MatrixInputs(f"case{seed}", N, K, W, bits, prow, pcol, idx, 0)


def lattice_case(N: int, K: int, seed: int, dist: Dict[int, float] | None = None,
                 x_range: int = 8) -> Tuple[MatrixInputs, np.ndarray]:
    """Integer-lattice weights: in the REORDERED frame every group of a b-bit
    block holds integers in [-2^(b-1), 2^(b-1)-1] and contains both extremes.
    0-bit blocks hold random normals (they are pruned).  Returns the inputs
    and a generator of integer activations in [-x_range, x_range]."""
    dist = DIST_SMOKE if dist is None else dist
    idx = 200 + seed
    g = rng(idx, 0, _ROLE_W)
    bits = draw_bits(N, K, dist, rng(idx, 0, _ROLE_BITS))
    prow = draw_perm(N, rng(idx, 0, _ROLE_PROW))
    pcol = draw_perm(K, rng(idx, 0, _ROLE_PCOL))
    wr = g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    brow = np.repeat(np.repeat(bits, BLOCK_ROWS, axis=0), BLOCK_COLS, axis=1).astype(np.int64)
    half = np.where(brow > 0, 1 << np.maximum(brow - 1, 0), 0)
    ints = g.integers(0, 1 << 30, size=(N, K)) % np.maximum(2 * half, 1) - half
    wr = np.where(brow > 0, ints.astype(np.float32), wr)
    # force both extremes into every group, at two distinct positions per group
    G = K // BLOCK_COLS
    p_lo = g.integers(0, BLOCK_COLS, size=(N, G))
    p_hi = (p_lo + 1 + g.integers(0, BLOCK_COLS - 1, size=(N, G))) % BLOCK_COLS
    rows = np.repeat(np.arange(N)[:, None], G, axis=1)
    base = BLOCK_COLS * np.arange(G)[None, :]
    b = bits[rows // BLOCK_ROWS, (p_lo + base) // BLOCK_COLS].astype(np.int64)
    h = np.where(b > 0, 1 << np.maximum(b - 1, 0), 0)
    sel = b > 0
    wr[rows[sel], (p_lo + base)[sel]] = (-h).astype(np.float32)[sel]
    wr[rows[sel], (p_hi + base)[sel]] = (h - 1).astype(np.float32)[sel]
    W = np.empty((N, K), dtype=np.float32)
    W[np.ix_(prow, pcol)] = wr
    mi = MatrixInputs(f"lattice{seed}", N, K, f32_to_bf16_bits(W), bits, prow, pcol, idx, 0)

    def xgen(M: int) -> np.ndarray:
        gx = rng(idx, 0, _ROLE_X, M)
        return f32_to_bf16_bits(gx.integers(-x_range, x_range + 1, size=(M, K)).astype(np.float32))

    return mi, xgen


# ---- synthetic block scores for the bit allocation --------------------------------------

ALLOC_LEVELS = (0, 1, 2, 3, 4, 8)


def draw_alloc_utility(n_blocks: int, seed: int, sigma: float = 1.5,
                       lo: float = 1e-3, hi: float = 1e3) -> np.ndarray:
    """Per-block utilities u[i][l] (fp32, [n_blocks][6]) for bitwidths 0, 1, 2, 3, 4, 8:
    u = -w_i * 4^-b, the expected squared RTN error of a block whose sensitivity w_i
    is log-normal (clipped to [lo, hi]); the error falls 4x per added bit.  A
    stand-in for the pages' first-order sensitivities, which need trained weights."""
    g = np.random.default_rng([0xA110C, seed])
    w = np.clip(np.exp(g.normal(0.0, sigma, n_blocks)), lo, hi)
    b = np.asarray(ALLOC_LEVELS, dtype=np.float64)
    return (-w[:, None] * np.power(4.0, -b)[None, :]).astype(np.float32)


def draw_saliency(N: int, K: int, seed: int, integer: bool = False) -> np.ndarray:
    """Per-weight saliency S[n][k] >= 0, fp32 [N][K]: w^2 * a_k^2 with w ~ N(0, 1) and
    per-column activation scales a_k log-normal (sigma 1), the usual activation-aware
    stand-in for the pages' sensitivities; `integer` gives small integers 0..15 (row
    and column sums then exact in fp32 in any order)."""
    g = np.random.default_rng([0x5A11, seed])
    if integer:
        return g.integers(0, 16, (N, K)).astype(np.float32)
    a = np.exp(g.normal(0.0, 1.0, K))
    w = g.standard_normal((N, K))
    return (w * w * (a * a)[None, :]).astype(np.float32)
