"""Bank model of the LDS tile layouts the gfx950 kernels use (no GPU needed).

LDS has 64 four-byte banks. A 16-byte-per-lane read (ds_read_b128) is served
16 lanes at a time, an 8-byte transposing read (ds_read_b64_tr_b16) 32 lanes at
a time; lanes of one group that hit the same bank at different addresses
conflict. For each layout this checks, on the index arithmetic the kernels
use, that
  * the direct-to-LDS writer puts every (row, 16-byte chunk) where the readers
    look for it, inside the tile;
  * the row-wise and transposing read patterns are conflict-free (the d=64
    forward V tile is the one known exception: it stays padded and 2-way
    conflicted, which the model must show).
The counters agree: SQ_LDS_BANK_CONFLICT reads 0 for every d=128 kernel.
"""
import pytest

BANKS = 64


def conflict_free(addrs, group):
    """addrs[lane] = list of dword addresses the lane touches."""
    for g0 in range(0, len(addrs), group):
        seen = {}
        for lane in range(g0, g0 + group):
            for dw in addrs[lane]:
                b = dw % BANKS
                if seen.get(b, dw) != dw:
                    return False
                seen[b] = dw
    return True


def writer_map(rows, stride, d, phys_to_logical):
    """Element offset -> (row, logical chunk) for a 1 KB-per-instruction
    direct-to-LDS writer over a tile of `rows` rows of `stride` elements;
    lanes in the padding write nothing."""
    held = {}
    for blk in range(rows * stride * 2 // 1024):
        for lane in range(64):
            off = blk * 1024 + lane * 16
            row, pc = off // (stride * 2), (off % (stride * 2)) >> 4
            if pc < d // 8:
                held[off // 2] = (row, phys_to_logical(row, pc))
    assert max(held) + 8 <= rows * stride
    return held


def tr_lane(lane):
    g = lane >> 5
    return 4 * g + ((lane & 15) >> 2), 16 * ((lane >> 4) & 1) + 4 * (lane & 3)


@pytest.mark.parametrize("d", [64, 128])
def test_xpad_tiles_both_read_patterns(d):
    """Backward Q/dO (dK/dV kernel) and K (dQ kernel) tiles: rows padded to a
    16-bank step, chunk c of row r at c ^ ((r >> 2) & 3)."""
    S, rows = d + 32, 64
    held = writer_map(rows, S, d, lambda r, pc: pc ^ ((r >> 2) & 3))
    for qt in range(rows // 32):
        for kk in range(d // 16):
            addrs = []
            for lane in range(64):
                r, g = lane & 31, lane >> 5
                xr = (r >> 2) & 3
                rw = (r * S + 8 * (g ^ xr), r * S + 8 * ((2 + g) ^ xr))
                e = 32 * qt * S + 32 * (kk >> 1) + rw[kk & 1]
                assert held[e] == (32 * qt + r, 2 * kk + g)
                addrs.append([e // 2 + i for i in range(4)])
            assert conflict_free(addrs, 16)
    for c in range(rows // 16):
        for t in range(d // 32):
            for j in range(2):
                addrs = []
                for lane in range(64):
                    g = lane >> 5
                    tr_row, tr_col = tr_lane(lane)
                    tw = (tr_row + 8 * j) * S + 8 * ((tr_col >> 3) ^ g ^ (2 * j)) + (tr_col & 7)
                    e = 16 * c * S + 32 * t + tw
                    assert held[e - e % 8] == (16 * c + tr_row + 8 * j, (32 * t + tr_col) >> 3)
                    addrs.append([e // 2, e // 2 + 1])
                assert conflict_free(addrs, 32)


def swz128(r):
    return ((r & 3) << 2) | ((r >> 2) & 3)


def test_forward_k_tile_swizzled():
    """d=128 forward K tile: unpadded, chunk c of row r at c ^ swz(r); row reads."""
    d, rows = 128, 64
    held = {}
    for blk in range(rows * d * 2 // 1024):
        for lane in range(64):
            e0 = blk * 512 + lane * 8
            row, pc = e0 // d, (e0 % d) >> 3
            held[e0] = (row, pc ^ swz128(row))
    for mt in range(rows // 32):
        for kk in range(d // 16):
            addrs = []
            for lane in range(64):
                r, g = lane & 31, lane >> 5
                col = 16 * kk + 8 * g
                e = 32 * mt * d + r * d + ((((col >> 3) ^ swz128(r)) << 3) | (col & 7))
                assert held[e] == (32 * mt + r, 2 * kk + g)
                addrs.append([e // 2 + i for i in range(4)])
            assert conflict_free(addrs, 16)


def test_forward_v_tile_xor_permuted():
    """d=128 forward V tile: unpadded, chunk c of row r at c ^ 4(r & 3);
    transposing reads with the lane's column group t at t ^ ((lane >> 2) & 3)."""
    d, rows = 128, 64
    held = {}
    for blk in range(rows * d * 2 // 1024):
        for lane in range(64):
            row, pc = blk * 4 + (lane >> 4), lane & 15
            held[blk * 512 + lane * 8] = (row, pc ^ (4 * (row & 3)))
    for c in range(rows // 16):
        for t in range(d // 32):
            for j in range(2):
                addrs = []
                for lane in range(64):
                    tr_row, tr_col = tr_lane(lane)
                    e = 16 * c * d + 8 * j * d + tr_row * d + tr_col + 32 * (t ^ ((lane >> 2) & 3))
                    col = 32 * t + tr_col
                    assert held[e - e % 8] == (16 * c + tr_row + 8 * j, col >> 3) and e % 8 == col % 8
                    addrs.append([e // 2, e // 2 + 1])
                assert conflict_free(addrs, 32)


def _padded_tr_conflict_free(stride, d, rows=64):
    for c in range(rows // 16):
        for t in range(d // 32):
            for j in range(2):
                addrs = []
                for lane in range(64):
                    tr_row, tr_col = tr_lane(lane)
                    e = (16 * c + tr_row + 8 * j) * stride + 32 * t + tr_col
                    addrs.append([e // 2, e // 2 + 1])
                if not conflict_free(addrs, 32):
                    return False
    return True


def test_padding_alone_cannot_serve_both_patterns():
    """Why the xpad XOR exists: the earlier 12-bank padding of the backward
    tiles, and the d=64 forward V stride, leave the transposing reads
    conflicted, while a plain 16-bank step breaks the row reads."""
    assert not _padded_tr_conflict_free(128 + 24, 128)
    assert not _padded_tr_conflict_free(64 + 8, 64)   # d=64 forward V tile (kept: no measurable cost)
    assert _padded_tr_conflict_free(128 + 32, 128)
    rows16 = [[(r * (128 + 32)) // 2 + i for i in range(4)] for r in range(16)]
    assert not conflict_free(rows16, 16)
