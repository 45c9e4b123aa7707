"""CPU oracle: block-wise mixed-precision weight-only quantized matmul.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in oracle/.  The
library (block_wise_mixed_amd) never does, and this file imports nothing from
it: the oracle and the HIP path share no code, no tables and no constants.
It is plain numpy, written from the definition of the method, and slow on
purpose where that keeps it checkable by eye.

What it computes, step by step
------------------------------
1. validate      -- shapes, bit values, permutations, finite weights.
2. reorder       -- Wr[i][j] = W[perm_row[i]][perm_col[j]]: rows and columns
                    reordered in both directions ("ScaleBITS" summary page,
                    section Approach; "SFMP" abstract, row-column reordering).
3. group_params  -- one asymmetric RTN group of 128 along K per row per
                    64x128 block ("ScaleBITS" summary page, sections Approach
                    and Limitations: RTN with group size 128), scale and zero
                    point in IEEE fp32 with a rounding after every operation.
4. quantize_codes-- q = clamp(rint(w / s) + z, 0, 2^b - 1), rint = half to even.
5. block_offsets -- exclusive prefix sum of bits over the packed order
                    (segments b = 1,2,3,4,8, row-major inside), in KiB.
6. pack / unpack -- the version-1 bit layout (one compact buffer, "TileQuant"
                    abstract: the precision map guides reconstruction into
                    compact weight buffers).
7. dequantize    -- W-hat = s * (q - z) in fp64 (exact).
8. matmul        -- y = x . W-hat^T in fp64, x gathered through perm_col, y
                    scattered back through perm_row so it is in original row
                    order.

16-bit blocks ("TileQuant" abstract: tiles kept at 16 bits beside 8-bit
ones) are a passthrough: the codes are the bf16 bit patterns of the reordered
weights in the same layout (one fragment per 1 KiB chunk), s = z = 0, and
W-hat is the bf16 weight itself (format version 2 = version 1 plus these
blocks; pinned by the identity W-hat == W and the bit-by-bit packer).

Readings where the pages are silent (all stated in the library header too):
64 rows along N x 128 columns along K per block; asymmetric RTN with the range
widened to include 0 (lo = min(0, min w), hi = max(0, max w)); integer zero
point z stored as uint8; ties to even; fp32 scale; 0-bit blocks are pruned
(s = z = 0, W-hat = 0); gather convention for permutations; y in fp32 on the
device, fp64 here.

Pins (tests/test_oracle_*.py check each of these against something other
than this file): quantizer bounds |w - W-hat| <= s/2 (+fp32 slack), 8-bit
within one step, 0-bit exactly zero; nearest level by brute force over all
2^b levels; the integer lattice where s = 1 and W-hat = W exactly; a worked
tie example; scale and zero equal to torch's per-channel min/max observer and
codes equal to torch's per-channel fake quantization; packing against an
independent bit-by-bit packer and round trip; y against a triple loop and
permutation invariances.  The choice of the bit layout itself has no page to
pin it to and is checked only for self-consistency ("parity unpinned" for
the layout choice, not for the values it stores).
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

BLOCK_ROWS = 64
BLOCK_COLS = 128
ALLOWED_BITS = (0, 1, 2, 3, 4, 8, 16)
SEGMENT_ORDER = (1, 2, 3, 4, 8, 16)
PASSTHROUGH_BITS = 16
NO_BLOCK = 0xFFFFFFFF
FORMAT_VERSION = 2


# --------------------------------------------------------------------------- inputs

def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def validate(N: int, K: int, bits: np.ndarray, perm_row: np.ndarray, perm_col: np.ndarray,
             W_f32: np.ndarray | None = None) -> None:
    """Raise ValueError if the problem is outside the method's domain."""
    if N <= 0 or K <= 0 or N % BLOCK_ROWS or K % BLOCK_COLS:
        raise ValueError(f"N={N} must be a positive multiple of 64 and K={K} of 128")
    bits = np.asarray(bits)
    if bits.shape != (N // BLOCK_ROWS, K // BLOCK_COLS):
        raise ValueError(f"bits shape {bits.shape} != {(N // BLOCK_ROWS, K // BLOCK_COLS)}")
    if not np.isin(bits, ALLOWED_BITS).all():
        raise ValueError("bits must be in {0,1,2,3,4,8,16}")
    for name, p, n in (("perm_row", perm_row, N), ("perm_col", perm_col, K)):
        p = np.asarray(p)
        if p.shape != (n,) or not np.array_equal(np.sort(p), np.arange(n)):
            raise ValueError(f"{name} is not a permutation of 0..{n - 1}")
    if W_f32 is not None:
        if not np.isfinite(W_f32).all() or (np.abs(W_f32) >= np.float32(2.0 ** 127)).any():
            raise ValueError("W must be finite with |W| < 2^127")


def reorder(W_f32: np.ndarray, perm_row: np.ndarray, perm_col: np.ndarray) -> np.ndarray:
    """Wr[i][j] = W[perm_row[i]][perm_col[j]] (gather convention)."""
    return np.ascontiguousarray(W_f32[np.asarray(perm_row)][:, np.asarray(perm_col)])


def row_bits(bits: np.ndarray) -> np.ndarray:
    """Bitwidth of every (row, group): [rows][K/128]."""
    return np.repeat(np.asarray(bits, dtype=np.int64), BLOCK_ROWS, axis=0)


# --------------------------------------------------------------------------- quantizer

def group_params(Wr: np.ndarray, bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Asymmetric RTN parameters of every (row, 128-group), fp32 with a rounding per op.

    Wr: float32 [R][K] reordered rows (R a multiple of 64); bits: [R/64][K/128].
    Returns scale float32 [R][K/128] and zero uint8 [R][K/128]:
        lo = min(0, min g), hi = max(0, max g), qmax = 2^b - 1,
        s = fl(fl(hi - lo) / qmax), z = clamp(rint(fl(-lo / s)), 0, qmax);
        b == 0 or s == 0 gives s = 0, z = 0.
    """
    Wr = np.asarray(Wr, dtype=np.float32)
    R, K = Wr.shape
    G = K // BLOCK_COLS
    g = Wr.reshape(R, G, BLOCK_COLS)
    lo = np.minimum(np.float32(0.0), g.min(axis=2))
    hi = np.maximum(np.float32(0.0), g.max(axis=2))
    b = row_bits(bits)
    qmax = (np.left_shift(1, b) - 1).astype(np.float32)
    live = (b > 0) & (b != PASSTHROUGH_BITS)  # 16-bit blocks keep bf16 values: s = z = 0
    d = (hi - lo).astype(np.float32)
    s = np.zeros((R, G), dtype=np.float32)
    s[live] = d[live] / qmax[live]
    z = np.zeros((R, G), dtype=np.float32)
    nz = s > 0
    zq = np.rint((-lo[nz]) / s[nz])
    z[nz] = np.minimum(np.maximum(zq, np.float32(0.0)), qmax[nz])
    return s, z.astype(np.uint8)


def quantize_codes(Wr: np.ndarray, bits: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Codes q = clamp(rint(fl(w / s)) + z, 0, qmax) as uint16 [R][K]; 0 where s == 0;
    in 16-bit blocks the bf16 bit pattern of w itself (passthrough, "TileQuant"
    abstract: tiles kept at 16 bits)."""
    Wr = np.asarray(Wr, dtype=np.float32)
    R, K = Wr.shape
    G = K // BLOCK_COLS
    out = _rtn_codes(Wr, bits, s, z).astype(np.uint16)
    pt = np.repeat(row_bits(bits) == PASSTHROUGH_BITS, BLOCK_COLS, axis=1)
    out[pt] = (Wr.view(np.uint32)[pt] >> 16).astype(np.uint16)
    return out


def _rtn_codes(Wr: np.ndarray, bits: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    R, K = Wr.shape
    G = K // BLOCK_COLS
    g = Wr.reshape(R, G, BLOCK_COLS)
    qmax = (np.left_shift(1, row_bits(bits)) - 1).astype(np.float32)
    q = np.zeros((R, G, BLOCK_COLS), dtype=np.float32)
    nz = s > 0
    t = np.rint(g[nz] / s[nz][:, None]) + z[nz].astype(np.float32)[:, None]
    q[nz] = np.minimum(np.maximum(t, np.float32(0.0)), qmax[nz][:, None])
    return q.astype(np.uint8).reshape(R, K)


def to_block_layout(a: np.ndarray) -> np.ndarray:
    """[R][G] per-(row, group) values -> [R/64][G][64] (block row, block col, row in block)."""
    R, G = a.shape
    return np.ascontiguousarray(a.reshape(R // BLOCK_ROWS, BLOCK_ROWS, G).transpose(0, 2, 1))


def from_block_layout(a: np.ndarray) -> np.ndarray:
    nbr, G, _ = a.shape
    return np.ascontiguousarray(a.transpose(0, 2, 1).reshape(nbr * BLOCK_ROWS, G))


# --------------------------------------------------------------------------- packed layout

def block_offsets(bits: np.ndarray) -> Tuple[np.ndarray, int]:
    """Exclusive prefix sum of bits over the packed order, in KiB.

    Packed order: segment b = 1, then 2, 3, 4, 8; row-major (r, c) inside a
    segment.  0-bit blocks get NO_BLOCK.  Returns (offsets uint32, code_bytes).
    """
    bits = np.asarray(bits)
    off = np.full(bits.shape, NO_BLOCK, dtype=np.uint32)
    total = 0
    for b in SEGMENT_ORDER:
        rs, cs = np.nonzero(bits == b)          # row-major order
        off[rs, cs] = total + b * np.arange(rs.size, dtype=np.int64)
        total += b * rs.size
    return off, 1024 * total


def _layout_maps(b: int) -> Tuple[np.ndarray, np.ndarray]:
    """For a {1,2,4,8}-bit block: word index and bit shift of every element [64][128]."""
    ib = np.arange(BLOCK_ROWS)[:, None]
    jb = np.arange(BLOCK_COLS)[None, :]
    rt, n = ib >> 4, ib & 15
    kt, kg, e = jb >> 5, (jb >> 3) & 3, jb & 7
    lane = n + 16 * kg
    F = 4 * rt + kt
    d, h = e >> 1, e & 1
    phi = 16 // b
    t, s = F // phi, F % phi
    byte = 1024 * t + 16 * lane + 4 * d
    return (byte // 4).astype(np.int64), (16 * h + b * s).astype(np.uint32)


_MAPS: Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}


def _sorted_maps(b: int):
    if b not in _MAPS:
        widx, shift = _layout_maps(b)
        order = np.argsort(widx.ravel(), kind="stable")
        _MAPS[b] = (order, shift.ravel()[order], widx.ravel()[order])
    return _MAPS[b]


def _pack_plane(q: np.ndarray, b: int) -> np.ndarray:
    """q [nblk][64][128] codes < 2^b -> uint32 words [nblk][256*b] (b in 1,2,4,8)."""
    order, shift, _ = _sorted_maps(b)
    nblk = q.shape[0]
    v = q.reshape(nblk, -1)[:, order].astype(np.uint32) << shift[None, :]
    # every word receives 32/b non-overlapping fields: their sum is their OR
    return v.reshape(nblk, 256 * b, 32 // b).sum(axis=2, dtype=np.uint64).astype(np.uint32)


def _unpack_plane(words: np.ndarray, b: int) -> np.ndarray:
    widx, shift = _layout_maps(b)
    nblk = words.shape[0]
    return ((words[:, widx.ravel()] >> shift.ravel()[None, :]) & np.uint32((1 << b) - 1)) \
        .astype(np.uint16 if b == PASSTHROUGH_BITS else np.uint8).reshape(nblk, BLOCK_ROWS, BLOCK_COLS)


def pack_blocks(q_blocks: np.ndarray, b: int) -> np.ndarray:
    """Bytes of b-bit blocks: q_blocks [nblk][64][128] -> uint8 [nblk][1024*b]."""
    q_blocks = np.asarray(q_blocks, dtype=np.uint16 if b == PASSTHROUGH_BITS else np.uint8)
    if b == 3:
        words = np.concatenate([_pack_plane(q_blocks & 3, 2), _pack_plane(q_blocks >> 2, 1)], axis=1)
    else:
        words = _pack_plane(q_blocks, b)
    return np.ascontiguousarray(words.astype("<u4")).view(np.uint8).reshape(q_blocks.shape[0], 1024 * b)


def unpack_blocks(raw: np.ndarray, b: int) -> np.ndarray:
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    words = raw.reshape(raw.shape[0], -1).view("<u4").astype(np.uint32)
    if b == 3:
        return _unpack_plane(words[:, :512], 2) | (_unpack_plane(words[:, 512:], 1) << 2)
    return _unpack_plane(words, b)


def blocks_of(q: np.ndarray) -> np.ndarray:
    """[R][K] -> [R/64][K/128][64][128]."""
    R, K = q.shape
    return q.reshape(R // BLOCK_ROWS, BLOCK_ROWS, K // BLOCK_COLS, BLOCK_COLS).transpose(0, 2, 1, 3)


def pack(q: np.ndarray, bits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Whole packed buffer: returns (block_offset uint32, codes uint8[code_bytes])."""
    off, code_bytes = block_offsets(bits)
    codes = np.zeros(code_bytes, dtype=np.uint8)
    qb = blocks_of(q)
    for b in SEGMENT_ORDER:
        rs, cs = np.nonzero(bits == b)
        if rs.size == 0:
            continue
        raw = pack_blocks(qb[rs, cs], b)
        start = off[rs, cs].astype(np.int64) * 1024
        idx = start[:, None] + np.arange(1024 * b)[None, :]
        codes[idx] = raw
    return off, codes


def unpack(codes: np.ndarray, bits: np.ndarray, off: np.ndarray) -> np.ndarray:
    """Inverse of pack: codes [N][K] (0 in 0-bit blocks)."""
    nbr, nbc = bits.shape
    q = np.zeros((nbr, nbc, BLOCK_ROWS, BLOCK_COLS), dtype=np.uint16)
    for b in SEGMENT_ORDER:
        rs, cs = np.nonzero(bits == b)
        if rs.size == 0:
            continue
        start = off[rs, cs].astype(np.int64) * 1024
        raw = codes[start[:, None] + np.arange(1024 * b)[None, :]]
        q[rs, cs] = unpack_blocks(raw, b)
    return np.ascontiguousarray(q.transpose(0, 2, 1, 3).reshape(nbr * BLOCK_ROWS, nbc * BLOCK_COLS))


# --------------------------------------------------------------------------- product

def dequantize(q: np.ndarray, s: np.ndarray, z: np.ndarray,
               bits: np.ndarray | None = None) -> np.ndarray:
    """W-hat[i][j] = s[i][j/128] * (q[i][j] - z[i][j/128]) in fp64 (exact); in 16-bit
    blocks (bits given) the bf16 value whose bit pattern q holds."""
    R, K = q.shape
    G = K // BLOCK_COLS
    qd = q.astype(np.float64).reshape(R, G, BLOCK_COLS) - z.astype(np.float64)[:, :, None]
    out = (s.astype(np.float64)[:, :, None] * qd).reshape(R, K)
    if bits is not None:
        pt = np.repeat(row_bits(bits) == PASSTHROUGH_BITS, BLOCK_COLS, axis=1)
        out[pt] = bf16_to_f32(np.asarray(q, dtype=np.uint16)[pt]).astype(np.float64)
    return out


def matmul(x_f32: np.ndarray, What_r: np.ndarray, perm_col: np.ndarray,
           perm_row: np.ndarray | None = None) -> np.ndarray:
    """y = x[:, perm_col] . What_r^T in fp64.

    What_r holds reordered rows.  With perm_row (all N rows covered) the result
    is scattered back to original row order: y[m][perm_row[i]] = yr[m][i].
    Without it the columns of the result follow the rows of What_r.
    """
    xr = np.asarray(x_f32, dtype=np.float64)[:, np.asarray(perm_col)]
    yr = xr @ np.asarray(What_r, dtype=np.float64).T
    if perm_row is None:
        return yr
    y = np.empty_like(yr)
    y[:, np.asarray(perm_row)] = yr
    return y


# --------------------------------------------------------------------------- one-call helpers

def quantize(W_bits: np.ndarray, bits: np.ndarray, perm_row: np.ndarray, perm_col: np.ndarray,
             block_rows: np.ndarray | None = None, check: bool = True) -> dict:
    """Steps 1-4 for all block rows, or for the listed reordered block rows only.

    Returns dict(rows, s [R][G], z [R][G], q [R][K], scale/zero in block layout
    [nbr][G][64], bits of the covered block rows)."""
    bits = np.asarray(bits)
    N, K = np.asarray(W_bits).shape
    W = bf16_to_f32(W_bits)
    if check:
        validate(N, K, bits, perm_row, perm_col, W)
    brs = np.arange(N // BLOCK_ROWS) if block_rows is None else np.asarray(block_rows)
    rows = (brs[:, None] * BLOCK_ROWS + np.arange(BLOCK_ROWS)[None, :]).ravel()
    Wr = reorder(W, np.asarray(perm_row)[rows], perm_col)
    sub_bits = bits[brs]
    s, z = group_params(Wr, sub_bits)
    q = quantize_codes(Wr, sub_bits, s, z)
    return dict(block_rows=brs, rows=rows, Wr=Wr, s=s, z=z, q=q, bits=sub_bits,
                scale=to_block_layout(s), zero=to_block_layout(z))


def quantize_pack(W_bits, bits, perm_row, perm_col) -> dict:
    """All of steps 1-6 for a whole matrix."""
    res = quantize(W_bits, bits, perm_row, perm_col)
    off, codes = pack(res["q"], np.asarray(bits))
    res.update(block_offset=off, codes=codes, code_bytes=int(codes.size))
    return res


def reference_gemm(x_bits: np.ndarray, qres: dict, perm_row: np.ndarray,
                   perm_col: np.ndarray) -> np.ndarray:
    """y_ref (fp64) from a quantize() result.

    All block rows covered: [M][N] in original row order.  A subset of block
    rows: [M][len(rows)], column t belonging to original output row
    perm_row[qres['rows'][t]]."""
    What = dequantize(qres["q"], qres["s"], qres["z"], qres["bits"])
    K = What.shape[1]
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16).reshape(-1, K))
    if What.shape[0] == len(perm_row):
        return matmul(x, What, perm_col, perm_row)
    return matmul(x, What, perm_col)
