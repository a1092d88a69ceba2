"""Helpers for the GPU parity tests: host <-> device marshalling and the
BF16 one-ulp comparison."""
from __future__ import annotations

import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(ref_bits: np.ndarray) -> np.ndarray:
    """ulp of each BF16 value: 2^(floor(log2|y|) - 7) for normal values, 2^-133 otherwise."""
    exp = ((ref_bits >> 7) & 0xFF).astype(np.int64)
    e = np.where(exp == 0, -126, exp - 127)
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def assert_bf16_within_1ulp(got_bits: np.ndarray, ref_bits: np.ndarray, what: str) -> int:
    """Assert |got - ref| <= ulp(ref) elementwise; return the count of non-identical values."""
    got_bits = np.asarray(got_bits).reshape(-1)
    ref_bits = np.asarray(ref_bits).reshape(-1)
    same = got_bits == ref_bits
    n_diff = int((~same).sum())
    if n_diff:
        g = bf16_to_f64(got_bits[~same])
        r = bf16_to_f64(ref_bits[~same])
        u = bf16_ulp(ref_bits[~same])
        bad = ~(np.abs(g - r) <= u)
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise AssertionError(f"{what}: {int(bad.sum())} values beyond 1 BF16 ulp "
                                 f"(first: got {g[i]!r} want {r[i]!r})")
    return n_diff
