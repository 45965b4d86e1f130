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


# ---------------------------------------------------------------------------
# FP8 tiles: rows of d one-byte codes, stored in the format of d/2 two-byte
# values (row bytes RB = d; RB = 64 uses swz(row) = (row >> 2) & 3).
# ---------------------------------------------------------------------------

def swz_bytes(RB, row):
    if RB == 64:
        return (row >> 2) & 3
    return swz(RB // 2, row)


def off_bytes(RB, row, chunk):
    return row * RB + ((chunk ^ swz_bytes(RB, row)) << 4)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_score_operand_reads_conflict_free(d):
    # K rows for the 8-bit score product j = kb + 2 kk: lane (r, g) reads row
    # 32 kb + r, chunks 4 kk + 2 g + h with two ds_read_b128 (h = 0, 1); the
    # kernel forms the address as row base + ((4 kk + h) ^ ((2 g) ^ swz(r))) << 4
    for kk in range(d // 64):
        for kb in range(2):
            for h in range(2):
                for lo in range(0, 64, 16):
                    banks = set()
                    for lane in range(lo, lo + 16):
                        r, g = lane & 31, lane >> 5
                        a = off_bytes(d, 32 * kb + r, 4 * kk + 2 * g + h)
                        short = (32 * kb + r) * d + (((4 * kk + h) ^ ((2 * g) ^ swz_bytes(d, r))) << 4)
                        assert a == short
                        banks |= {(a // 4 + i) % 64 for i in range(4)}
                    assert len(banks) == 64, (d, kk, kb, h, lo)


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_transposed_value_reads(d):
    # ds_read_b64_tr_b8 for output block db, read t: the lane pair 2e, 2e+1 of a
    # 16-lane group addresses row 32 (t/2) + 16 (t%2) + 8 (e/4) + 4 g + e%4,
    # bytes 32 db + 16 gi + 8 (lane % 2) .. +7.  Checks: the kernel's short
    # address form, the rows each lane receives (the keys of P's register order),
    # and no bank conflict among the 32 lanes served per cycle.
    for db in range(d // 32):
        for t in range(4):
            for lo in (0, 32):
                banks = set()
                for lane in range(lo, lo + 32):
                    s16, gi, g = lane & 15, (lane >> 4) & 1, lane >> 5
                    e = s16 >> 1
                    vrl = 8 * (e >> 2) + 4 * g + (e & 3)
                    R = 32 * (t >> 1) + 16 * (t & 1) + vrl
                    col = 32 * db + 16 * gi + 8 * (s16 & 1)
                    a = off_bytes(d, R, col >> 4) + (col & 15)
                    short = (32 * (t >> 1) + 16 * (t & 1)) * d + vrl * d + 8 * (s16 & 1) \
                        + ((db << 5) ^ ((gi ^ swz_bytes(d, vrl)) << 4))
                    assert a == short
                    banks |= {(a // 4 + i) % 64 for i in range(2)}
                assert len(banks) == 64, (d, db, t, lo)
    # received rows: lane l of 16-lane group gets byte l % 8 of the piece of lane
    # 2e + l / 8, i.e. column col0 + l, rows R(e) for e = 0..7; byte j = 8 t + e of
    # lane group g must be key 32 (j / 16) + 8 ((j % 16) / 4) + 4 g + j % 4
    for g in range(2):
        for t in range(4):
            for e in range(8):
                j = 8 * t + e
                R = 32 * (t >> 1) + 16 * (t & 1) + 8 * (e >> 2) + 4 * g + (e & 3)
                assert R == 32 * (j // 16) + 8 * ((j % 16) // 4) + 4 * g + j % 4


# --- output staging (store_rows_staged) -------------------------------------
# A wavefront's 32 output rows go through a 32 x 2D-byte LDS area: lane
# r + 32 g writes 8 bytes per (column block db, quad qd) at row r, logical
# chunk db*4 + qd, half g; then lane l reads 16 bytes of row
# i * RPI + l // CPR, logical chunk l % CPR, and stores them to that row of
# the output.  Chunks are XOR-swizzled by the row's 256-byte bank line:
# row & 15 at D = 128, (row >> 1) & 7 at D = 64.

def stage_off(D, row, chunk):
    cpr = D // 8
    line = row if D == 128 else row >> 1
    return row * 2 * D + ((chunk ^ (line & (cpr - 1))) << 4)


@pytest.mark.parametrize("D", [64, 128])
def test_staged_rows_round_trip(D):
    # every (row, column) written by the accumulator layout is read back by
    # exactly one lane and lands in the same row and column of the output
    cpr, rpi = D // 8, 64 // (D // 8)
    lds = {}
    for lane in range(64):
        r, g = lane & 31, lane >> 5
        for db in range(D // 32):
            for qd in range(4):
                a = stage_off(D, r, db * 4 + qd) + g * 8
                for e in range(4):   # four bf16 values, columns db*32 + qd*8 + g*4 + e
                    col = db * 32 + qd * 8 + g * 4 + e
                    key = a + 2 * e
                    assert key not in lds
                    assert 0 <= key < 32 * 2 * D
                    lds[key] = (r, col)
    assert len(lds) == 32 * D
    seen = set()
    for i in range(32 // rpi):
        for lane in range(64):
            row, ch = i * rpi + lane // cpr, lane % cpr
            a = stage_off(D, row, ch)
            for e in range(8):   # 16 bytes = columns ch*8 .. ch*8+7 of the output row
                assert lds[a + 2 * e] == (row, ch * 8 + e)
                seen.add((row, ch * 8 + e))
    assert len(seen) == 32 * D


@pytest.mark.parametrize("D", [64, 128])
def test_staged_rows_bank_use(D):
    # ds_write_b64: each 32-lane half of an instruction (256 bytes) should
    # touch every bank at most twice; ds_read_b128: each 16-lane quarter
    # (256 bytes) at most once per 64 banks, i.e. distinct banks
    cpr, rpi = D // 8, 64 // (D // 8)
    for db in range(D // 32):
        for qd in range(4):
            for lo in (0, 32):
                count = {}
                for lane in range(lo, lo + 32):
                    r, g = lane & 31, lane >> 5
                    a = stage_off(D, r, db * 4 + qd) + g * 8
                    for w in range(2):
                        b = (a // 4 + w) % 64
                        count[b] = count.get(b, 0) + 1
                assert max(count.values()) <= 2
    for i in range(32 // rpi):
        for lo in range(0, 64, 16):
            banks = set()
            for lane in range(lo, lo + 16):
                row, ch = i * rpi + lane // cpr, lane % cpr
                a = stage_off(D, row, ch)
                for w in range(4):
                    banks.add((a // 4 + w) % 64)
            assert len(banks) == 64
