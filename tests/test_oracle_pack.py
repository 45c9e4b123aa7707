"""Pins of the oracle's packed layout and block-offset table.

The bit layout (format version 1) is this library's own choice; no page fixes
it, so it is checked for self-consistency: the oracle's vectorized packer
against an independent bit-by-bit packer written from the layout text, a round
trip, a bijection check and the sizes the layout implies.  The offset table is
pinned by its definition: exclusive prefix sum over the packed order
(segments b = 1,2,3,4,8, row-major inside), in KiB.
"""
import numpy as np
import pytest

import oracle
from block_wise_mixed_amd import synth


def slow_pack_block(q, b):
    """Bit-by-bit packer: for every element, place each code bit at its byte/bit address."""
    out = bytearray(1024 * b)

    def put(code, width, t_base, phi, ib, jb):
        rt, n = ib // 16, ib % 16
        kt, kg, e = jb // 32, (jb // 8) % 4, jb % 8
        lane = n + 16 * kg
        F = 4 * rt + kt
        d, h = e // 2, e % 2
        t, s = t_base + F // phi, F % phi
        bitpos = 16 * h + width * s
        for k in range(width):
            if (code >> k) & 1:
                p = bitpos + k
                out[1024 * t + 16 * lane + 4 * d + p // 8] |= 1 << (p % 8)

    for ib in range(64):
        for jb in range(128):
            v = int(q[ib][jb])
            if b == 3:
                put(v & 3, 2, 0, 8, ib, jb)
                put(v >> 2, 1, 2, 16, ib, jb)
            else:
                put(v, b, 0, 16 // b, ib, jb)
    return np.frombuffer(bytes(out), dtype=np.uint8)


@pytest.mark.parametrize("b", [1, 2, 3, 4, 8, 16])
def test_vectorized_pack_matches_bit_by_bit(b):
    g = np.random.default_rng(b)
    q = g.integers(0, 1 << b, size=(3, 64, 128)).astype(np.uint16 if b == 16 else np.uint8)
    fast = oracle.pack_blocks(q, b)
    for i in range(3):
        assert np.array_equal(fast[i], slow_pack_block(q[i], b))


def _bit_address(ib, jb, k, b):
    """Bit address (inside the block) of bit k of element (ib, jb), read off the layout text."""
    if b == 3:
        return _bit_address(ib, jb, k, 2) if k < 2 else 2 * 8192 + _bit_address(ib, jb, 0, 1)
    rt, n = ib // 16, ib % 16
    kt, kg, e = jb // 32, (jb // 8) % 4, jb % 8
    lane = n + 16 * kg
    F = 4 * rt + kt
    phi = 16 // b
    t, s = F // phi, F % phi
    byte = 1024 * t + 16 * lane + 4 * (e // 2)
    return 8 * byte + 16 * (e % 2) + b * s + k


@pytest.mark.parametrize("b", [1, 2, 3, 4, 8])
def test_layout_is_a_bijection(b):
    """Every code bit of the block has its own bit and the block is exactly 8192*b bits;
    the packer puts each single set bit where the layout text says."""
    addr = [_bit_address(ib, jb, k, b) for ib in range(64) for jb in range(128) for k in range(b)]
    assert sorted(addr) == list(range(8192 * b))
    g = np.random.default_rng(20 + b)
    for _ in range(16):
        ib, jb, k = int(g.integers(64)), int(g.integers(128)), int(g.integers(b))
        q = np.zeros((1, 64, 128), dtype=np.uint8)
        q[0, ib, jb] = 1 << k
        on = np.nonzero(np.unpackbits(oracle.pack_blocks(q, b)[0], bitorder="little"))[0]
        assert list(on) == [_bit_address(ib, jb, k, b)]


@pytest.mark.parametrize("b", [1, 2, 3, 4, 8, 16])
def test_unpack_inverts_pack(b):
    g = np.random.default_rng(10 + b)
    q = g.integers(0, 1 << b, size=(5, 64, 128)).astype(np.uint16 if b == 16 else np.uint8)
    assert np.array_equal(oracle.unpack_blocks(oracle.pack_blocks(q, b), b), q)


def test_chunk_is_mfma_fragment():
    """For b in {1,2,4,8}, masking the four words of one lane at one slot yields one row x
    8 consecutive columns (the 16x32 operand fragment the format is built around)."""
    for b in (1, 2, 4, 8):
        q = np.arange(64 * 128).reshape(1, 64, 128)
        # encode (ib, jb) coordinates one bit-plane at a time is heavy; instead check the map
        widx, shift = oracle.msq_oracle._layout_maps(b)
        phi = 16 // b
        for t in range(b):
            for lane in (0, 5, 17, 63):
                for s in range(phi):
                    rows_cols = set()
                    for d in range(4):
                        for h in range(2):
                            hit = np.nonzero((widx == 256 * t + 4 * lane + d) & (shift == 16 * h + b * s))
                            assert hit[0].size == 1
                            rows_cols.add((int(hit[0][0]), int(hit[1][0])))
                    rows = {r for r, _ in rows_cols}
                    cols = sorted(c for _, c in rows_cols)
                    assert len(rows) == 1
                    assert cols == list(range(cols[0], cols[0] + 8)) and cols[0] % 8 == 0
        del q


def test_offsets_are_prefix_sum_over_packed_order():
    g = np.random.default_rng(3)
    bits = g.choice(np.array([0, 1, 2, 3, 4, 8, 16], np.uint8), size=(7, 9))
    off, code_bytes = oracle.block_offsets(bits)
    assert code_bytes == 1024 * int(bits.astype(np.int64).sum())
    # brute force: walk the packed order explicitly
    acc = 0
    for b in (1, 2, 3, 4, 8, 16):
        for r in range(7):
            for c in range(9):
                if bits[r, c] == b:
                    assert off[r, c] == acc
                    acc += b
    assert (off[bits == 0] == 0xFFFFFFFF).all()
    assert acc * 1024 == code_bytes


def test_whole_buffer_round_trip_and_size():
    c = synth.random_case(320, 640, 7)
    r = oracle.quantize_pack(c.W, c.bits, c.perm_row, c.perm_col)
    assert r["codes"].size == 1024 * int(c.bits.astype(np.int64).sum())
    q = oracle.unpack(r["codes"], c.bits, r["block_offset"])
    assert np.array_equal(q, r["q"])
    # every byte of the buffer belongs to exactly one block
    owner = np.zeros(r["codes"].size, np.int64)
    for (rr, cc), b in np.ndenumerate(c.bits):
        if b:
            o = int(r["block_offset"][rr, cc]) * 1024
            owner[o:o + 1024 * int(b)] += 1
    assert (owner == 1).all()


def test_empty_segments_and_all_zero_bits():
    bits = np.zeros((2, 3), np.uint8)
    off, cb = oracle.block_offsets(bits)
    assert cb == 0 and (off == 0xFFFFFFFF).all()
    bits = np.full((2, 3), 8, np.uint8)
    off, cb = oracle.block_offsets(bits)
    assert cb == 6 * 8192 and list(off.ravel()) == [0, 8, 16, 24, 32, 40]


def test_passthrough_chunk_is_the_bf16_fragment():
    """16-bit blocks: chunk F holds, at lane l's 16 bytes, the eight bf16 values of row
    16 (F >> 2) + (l & 15), columns 32 (F & 3) + 8 (l >> 4) .. + 7, little-endian,
    i.e. the matrix-core B operand of that fragment with no unpacking."""
    g = np.random.default_rng(77)
    q = g.integers(0, 1 << 16, size=(1, 64, 128)).astype(np.uint16)
    raw = oracle.pack_blocks(q, 16)[0].view("<u2").reshape(16, 64, 8)
    for F in range(16):
        for l in range(64):
            row = 16 * (F >> 2) + (l & 15)
            col = 32 * (F & 3) + 8 * (l >> 4)
            assert np.array_equal(raw[F, l], q[0, row, col:col + 8])
