"""Host model of the LDS bank mapping of the transposing fragment reads (K x N tiles, and the
weight gradient's K x M A tile).

The model: a 64-lane ds_read_b64_tr_b16 is served in two 32-lane halves; LDS has 64 banks of
4 bytes, so a half reads 256 bytes and is conflict-free when its 32 lanes' 8-byte words cover
all 64 banks.  The swizzle and the per-lane address formulas below restate those of the
kernel sources (ptg_device.hpp: swz_n, consumer_role's and consumer_role16's read offsets)
for the tile widths in use; the counters of the profiled runs show the same result (zero
bank-conflict cycles).
"""
import pytest


def swz_n(k, cpr):
    m = k & 3
    return ((m & 1) * 6) ^ ((m & 2) * 5) ^ (((k >> 3) & 1) << 1) if cpr >= 16 else (k & 3) << 1


def banks(addrs):
    out = []
    for a in addrs:
        out += [(a // 4) % 64, (a // 4 + 1) % 64]
    return out


def read16(lane, row_len, w_first, blk, ks, second):
    """16x16x32 consumer: 16-lane group g reads k-rows 8 g + i / 4 (+ 4 for the second read)
    of slice ks, columns 4 (i % 4) .. + 3 of 16-column block blk of the wave's sub-tile."""
    g, i = lane >> 4, lane & 15
    k = g * 8 + (i >> 2) + (4 if second else 0) + ks * 32
    n = w_first + blk * 16 + (i & 3) * 4
    cpr = row_len // 8
    return k * row_len * 2 + (((n >> 3) ^ swz_n(k, cpr)) << 4) + ((n >> 2) & 1) * 8


def read32(lane, row_len, w_first, blk, kk, second):
    """32x32x16 consumer: 16-lane block b reads k-rows 8 (b / 2) + i / 4 (+ 4), columns
    16 (b % 2) + 4 (i % 4) .. + 3 of 32-column block blk."""
    b, i = lane >> 4, lane & 15
    k = (b >> 1) * 8 + (i >> 2) + (4 if second else 0) + kk * 16
    n = w_first + blk * 32 + (b & 1) * 16 + (i & 3) * 4
    cpr = row_len // 8
    return k * row_len * 2 + (((n >> 3) ^ swz_n(k, cpr)) << 4) + ((n >> 2) & 1) * 8


@pytest.mark.parametrize("row_len,wave_cols,blocks", [(256, 64, 4), (256, 128, 8)])
def test_16x16_transposing_reads_are_conflict_free(row_len, wave_cols, blocks):
    # row_len 256: B tile of 256 columns (waves of 64 columns) and A tile of 256 rows stored
    # K x M (waves of 128 rows, 8 blocks)
    for w in range(row_len // wave_cols):
        for blk in range(blocks):
            for ks in range(2):
                for second in (False, True):
                    addrs = [read16(l, row_len, w * wave_cols, blk, ks, second) for l in range(64)]
                    for half in (addrs[:32], addrs[32:]):
                        assert len(set(banks(half))) == 64, (w, blk, ks, second)


def test_32x32_transposing_reads_are_conflict_free():
    row_len, wave_cols = 128, 64       # medium tile: 128 columns, waves of 64 (2 blocks)
    for w in range(2):
        for blk in range(2):
            for kk in range(4):
                for second in (False, True):
                    addrs = [read32(l, row_len, w * wave_cols, blk, kk, second) for l in range(64)]
                    for half in (addrs[:32], addrs[32:]):
                        assert len(set(banks(half))) == 64


def test_swizzle_without_bit3_conflicts_in_16x16_reads():
    """The reason for the bit-3 term: with a swizzle of k mod 4 alone, the two 16-lane groups of
    a half read the same banks."""
    def old(k, cpr):
        m = k & 3
        return ((m & 1) * 6) ^ ((m & 2) * 5)
    g = globals()
    saved = g["swz_n"]
    try:
        g["swz_n"] = old
        addrs = [read16(l, 256, 0, 0, 0, False) for l in range(64)]
        assert len(set(banks(addrs[:32]))) == 32
    finally:
        g["swz_n"] = saved
