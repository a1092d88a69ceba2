"""The tests' FP6 operand-format decoder (tests/fp6_format.py) against the
OCP Microscaling formats specification's E2M3 values and a bit-by-bit
reading of the format description (CPU only)."""
from fractions import Fraction

import numpy as np

import fp6_format as F


def test_e2m3_values_from_the_specification():
    # E2M3: exponent bias 1, 3 mantissa bits, no infinities or NaN.
    assert F.e2m3_value(0b000000) == 0
    assert F.e2m3_value(0b000001) == Fraction(1, 8)      # smallest subnormal
    assert F.e2m3_value(0b000111) == Fraction(7, 8)      # largest subnormal
    assert F.e2m3_value(0b001000) == 1                   # smallest normal
    assert F.e2m3_value(0b010000) == 2
    assert F.e2m3_value(0b011000) == 4
    assert F.e2m3_value(0b011111) == Fraction(15, 2)     # largest normal, 7.5
    assert F.e2m3_value(0b111111) == Fraction(-15, 2)
    assert F.e2m3_value(0b101000) == -1
    mags = sorted({abs(F.e2m3_value(f)) for f in range(64)})
    assert len(mags) == 32 and mags[-1] == Fraction(15, 2)


def test_code_table():
    # each code in [-7, 7] has exactly one canonical field; 0 is +0
    for c in range(-7, 8):
        fields = np.flatnonzero(F.CODE_OF_FIELD == c)
        assert len(fields) == 1, c
        assert F.e2m3_value(int(fields[0])) == c
    assert F.CODE_OF_FIELD[0] == 0 and F.CODE_OF_FIELD[0b100000] == F.INVALID
    assert F.CODE_OF_FIELD[0b000100] == F.INVALID                   # 0.5
    assert F.CODE_OF_FIELD[0b011111] == F.INVALID                   # 7.5
    assert int((F.CODE_OF_FIELD != F.INVALID).sum()) == 15


def test_vectorised_decoder_matches_bitwise_reading():
    g = np.random.Generator(np.random.PCG64(41))
    R, K = 40, 192                                  # rows with every (bit 3, bit 4) pair
    packed = g.integers(0, 256, (R, 3 * K // 4), dtype=np.int64).astype(np.uint8)
    fields = F.decode_fields(packed, K)
    for r in range(R):
        slow = F.slow_decode_row(bytes(packed[r]), K, r)
        assert [F.e2m3_value(int(f)) for f in fields[r]] == slow, r
    # the row offset selects the tail order of the rows that follow
    assert np.array_equal(F.decode_fields(packed[8:24], K, row0=8), fields[8:24])


def test_hand_built_rows():
    # row 0 (tails in order): code 5 (field 0b011010) as value 37 = piece 1 value 5, bits 30..35
    row = np.zeros((1, 48), np.uint8)
    bits = 0b011010 << 30
    for i in range(24):
        byte = (bits >> (8 * i)) & 0xFF
        row[0, 16 + i if i < 16 else 40 + (i - 16)] = byte
    codes = F.decode_codes(row, 64)
    want = np.zeros((1, 64), np.int8)
    want[0, 37] = 5
    assert np.array_equal(codes, want)
    # row 8 (bits 3 and 4 differ): piece 1's tail comes first; -7 (0b111110) as value 63,
    # the last field of piece 1, bits 186..191 = tail byte 7 of piece 1 -> byte 39
    row8 = np.zeros((9, 48), np.uint8)
    row8[8, 39] = 0b111110 << 2
    codes = F.decode_codes(row8, 64)
    want = np.zeros((9, 64), np.int8)
    want[8, 63] = -7
    assert np.array_equal(codes, want)
    # the same bytes on row 0 belong to piece 0's tail (value 31)
    codes0 = F.decode_codes(row8[8:9], 64, row0=0)
    assert codes0[0, 31] == -7 and np.count_nonzero(codes0) == 1


def test_unslice96():
    g = np.random.Generator(np.random.PCG64(42))
    R, B = 5, 192
    rm = g.integers(0, 256, (R, B), dtype=np.int64).astype(np.uint8)
    sl = np.concatenate([rm[:, 96 * t:96 * (t + 1)].reshape(-1) for t in range(B // 96)])
    assert np.array_equal(F.unslice96(sl, R), rm)
