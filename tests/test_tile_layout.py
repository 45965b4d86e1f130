"""Host-side checks of the LDS tile layout the kernels rely on.

The kernels read the swizzled LDS tiles in two patterns and compute the two
addresses as (x ^ c) + a with a per-lane x and a, and a compile-time c; this test
re-derives both from the tile's definition (row-major rows of D bf16, 16-byte
chunks XOR-permuted within each row by swz(row)) and checks that the short forms
agree for every lane and step, and that both patterns are free of LDS bank
conflicts (each group of lanes served in one cycle touches distinct banks).
"""

import pytest


def swz(D, row):
    if D == 128:
        return ((row & 3) << 2) | ((row >> 2) & 3)
    return (((row >> 1) & 1) << 2) | ((row >> 2) & 3)


def off(D, row, chunk):
    return row * D * 2 + ((chunk ^ swz(D, row)) << 4)


def tr_offset(D, col0, lane, half):
    s, gi, g = lane & 15, (lane >> 4) & 1, lane >> 5
    row = half * 8 + g * 4 + (s >> 2)
    col = col0 + 16 * gi + 4 * (s & 3)
    return off(D, row, col >> 3) + ((col & 7) << 1)


@pytest.mark.parametrize("D", [64, 128])
def test_short_address_forms(D):
    for lane in range(64):
        r, g = lane & 31, lane >> 5
        ar, xr = r * D * 2, (g ^ swz(D, r)) << 4
        for kk in range(D // 16):
            assert off(D, r, 2 * kk + g) == ((xr ^ (kk << 5)) + ar)
        s, gi = lane & 15, (lane >> 4) & 1
        lo = 2 * gi + ((s & 3) >> 1)
        xts = set()
        for half in range(2):
            row = half * 8 + g * 4 + (s >> 2)
            sw = swz(D, row)
            at = row * D * 2 + ((lo ^ (sw & 3)) << 4) + ((s & 1) << 3)
            xt = (sw & ~3) << 4
            xts.add(xt)
            for db in range(D // 32):
                assert tr_offset(D, db * 32, lane, half) == ((xt ^ (db << 6)) + at)
        assert len(xts) == 1


@pytest.mark.parametrize("D", [64, 128])
def test_row_reads_conflict_free(D):
    # ds_read_b128: 16 lanes x 16 bytes per cycle must cover 64 distinct banks
    for kk in range(D // 16):
        for lo in range(0, 64, 16):
            banks = set()
            for lane in range(lo, lo + 16):
                r, g = lane & 31, lane >> 5
                a = off(D, r, 2 * kk + g)
                banks |= {(a // 4 + i) % 64 for i in range(4)}
            assert len(banks) == 64, (D, kk, lo)


@pytest.mark.parametrize("D", [64, 128])
def test_transposed_reads_conflict_free(D):
    # ds_read_b64_tr_b16: 32 lanes x 8 bytes per cycle must cover 64 distinct banks
    for db in range(D // 32):
        for half in range(2):
            for lo in (0, 32):
                banks = set()
                for lane in range(lo, lo + 32):
                    a = tr_offset(D, db * 32, lane, half)
                    banks |= {(a // 4 + i) % 64 for i in range(2)}
                assert len(banks) == 64, (D, db, half, lo)
