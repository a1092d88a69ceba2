"""The library's FP6 operand format, decoded from its description in the C
header (include/qdiff.h, "FP6 operand format"), for the GPU tests.

This is test infrastructure only.  The oracle knows nothing of the format:
it produces INT4 codes, and the tests decode the bytes the GPU writes back
into codes and compare those with the oracle's codes element by element.

The format, as the header states it, for an [R, K] matrix (K % 64 == 0):
each row takes 3K/4 bytes; values 64j .. 64j+63 fill the 48 bytes at 48j
as two pieces of 32 values (value i of a piece in bits 6i .. 6i+5 of the
piece's 24 bytes, least significant first); bytes 0..15 hold piece 0's
bytes 0..15, bytes 16..31 piece 1's bytes 0..15, and bytes 32..47 the two
pieces' 8-byte tails, piece 0's first unless bits 3 and 4 of the row index
differ.  A value is an FP6 E2M3 field of the OCP Microscaling formats
specification (sign bit 5, exponent bits 4..3 with bias 1, mantissa bits
2..0; exponent field 0 encodes m/8, otherwise 2^(e-1)(1 + m/8)), and the
code 0 is stored as +0.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

INVALID = -128   # decoded value that is not a code of [-7, 7] in its canonical field


def e2m3_value(f: int) -> Fraction:
    """The exact value of the 6-bit E2M3 field f."""
    s, e, m = (f >> 5) & 1, (f >> 3) & 3, f & 7
    mag = Fraction(m, 8) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 8))
    return -mag if s else mag


def _code_table() -> np.ndarray:
    """Field -> INT4 code, INVALID for a non-integer value, for a magnitude
    above 7, or for -0 (zero is stored as +0)."""
    t = np.full(64, INVALID, np.int8)
    for f in range(64):
        v = e2m3_value(f)
        if v.denominator == 1 and abs(v) <= 7 and f != 0b100000:
            t[f] = int(v)
    return t


CODE_OF_FIELD = _code_table()


def row_swaps(rows: np.ndarray) -> np.ndarray:
    """True for rows whose two 8-byte tails are stored piece 1 first."""
    rows = np.asarray(rows, np.int64)
    return (((rows >> 3) ^ (rows >> 4)) & 1).astype(bool)


def decode_fields(packed: np.ndarray, K: int, row0: int = 0) -> np.ndarray:
    """packed [R, >= 3K/4] uint8 (rows row0 .. row0 + R - 1 of the operand)
    -> the 6-bit fields [R, K] (uint8) in value order."""
    packed = np.asarray(packed, np.uint8)
    R = packed.shape[0]
    assert K % 64 == 0 and packed.shape[1] >= 3 * K // 4
    blk = packed[:, :3 * K // 4].reshape(R, K // 64, 48)
    sw = row_swaps(np.arange(row0, row0 + R))[:, None, None]
    tail0 = np.where(sw, blk[:, :, 40:48], blk[:, :, 32:40])
    tail1 = np.where(sw, blk[:, :, 32:40], blk[:, :, 40:48])
    p0 = np.concatenate([blk[:, :, 0:16], tail0], axis=2)          # [R, K/64, 24]
    p1 = np.concatenate([blk[:, :, 16:32], tail1], axis=2)
    g = np.stack([p0, p1], axis=2).reshape(R, K // 64, 2, 8, 3).astype(np.uint32)
    v = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)           # 4 fields per 3 bytes
    f = (v[..., None] >> (6 * np.arange(4, dtype=np.uint32))) & 63
    return f.reshape(R, K).astype(np.uint8)


def decode_codes(packed: np.ndarray, K: int, row0: int = 0) -> np.ndarray:
    """packed FP6 operand rows -> INT4 codes [R, K] int8 (INVALID where a
    field is not the canonical encoding of a code in [-7, 7])."""
    return CODE_OF_FIELD[decode_fields(packed, K, row0)]


def unslice96(b: np.ndarray, R: int) -> np.ndarray:
    """The K-sliced layout (byte b of row r at (b / 96) R 96 + r 96 + b % 96)
    -> row-major [R, 3K/4] bytes."""
    b = np.asarray(b, np.uint8).reshape(-1, R, 96)
    return np.ascontiguousarray(b.transpose(1, 0, 2)).reshape(R, -1)


def assert_fp6_codes(packed: np.ndarray, codes: np.ndarray, what: str, chunk: int = 512) -> None:
    """Every value of the FP6 operand rows `packed` decodes to the INT4 code
    in `codes` (same shape [R, K]), row chunk by row chunk."""
    codes = np.asarray(codes)
    R, K = codes.shape
    assert packed.shape[0] == R, (packed.shape, codes.shape)
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        got = decode_codes(packed[r0:r1], K, r0)
        if not np.array_equal(got, codes[r0:r1]):
            bad = np.argwhere(got != codes[r0:r1])
            r, k = bad[0]
            raise AssertionError(f"{what}: {len(bad)} FP6 values differ from the codes "
                                 f"(first at row {r0 + r}, k {k}: decoded {got[r, k]}, code {codes[r0 + r, k]})")


def slow_decode_row(row: bytes, K: int, r: int) -> list:
    """Exact values of one row, bit by bit from the description (reference
    for the vectorised decoder)."""
    vals = []
    for j in range(K // 64):
        blk = bytes(row[48 * j:48 * j + 48])
        first, second = blk[32:40], blk[40:48]
        t0, t1 = (second, first) if ((r >> 3) ^ (r >> 4)) & 1 else (first, second)
        for piece in (blk[0:16] + t0, blk[16:32] + t1):
            bits = int.from_bytes(piece, "little")
            for i in range(32):
                vals.append(e2m3_value((bits >> (6 * i)) & 63))
    return vals
