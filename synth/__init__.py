"""Seeded synthetic inputs for the rotated INT8 linear layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic (no rotation, no quantization, no GEMM).  Both the oracle
side (tests, CPU baseline) and the GPU side (tests, benchmark) take their
inputs from here, so the two always see the same bytes.

Workloads (the SGLang pull request "Tune Kitchen INT8 row splitting for
SM120", Benchmark & Profiling table and Modifications paragraph, gives the
M/K/N shapes; the dtypes are from its Accuracy Test paragraph):

  id  M      K      N      kind   outlier channels
  1   256    512    512    w8a8   4
  2   8193   5376   16128  w8a8   round(0.01*K) = 54
  3   32700  5376   16128  w8a8   54
  4   14850  7168   28672  w8a8   72
  5   8192   28672  7168   w4a4   287

Value recipe:
  x    ~ N(0, 1) in FP32, the outlier columns (chosen without replacement)
         multiplied by 20, then rounded to BF16 (round-to-nearest-even).
  W    ~ N(0, 0.02) in FP32, shape [N, K] (nn.Linear layout).
  bias ~ N(0, 0.1) in FP32, rounded to BF16.
Generators are NumPy PCG64 with seeds 1000+c (x), 2000+c (W), 3000+c (bias),
4000+c (outlier columns), c = workload id.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "make_x", "make_w", "make_bias", "iter_x", "iter_w",
           "outlier_columns", "f32_to_bf16_bits", "bf16_bits_to_f32", "random_bf16"]


@dataclass(frozen=True)
class Workload:
    cid: int
    M: int
    K: int
    N: int
    kind: str          # "w8a8" or "w4a4"
    n_outliers: int

    @property
    def name(self) -> str:
        tag = "INT8 linear" if self.kind == "w8a8" else "W4A4 rotated linear"
        return f"{tag} M{self.M}/K{self.K}/N{self.N}"


def _n_out(K: int) -> int:
    return int(round(0.01 * K))


WORKLOADS = {
    1: Workload(1, 256, 512, 512, "w8a8", 4),
    2: Workload(2, 8193, 5376, 16128, "w8a8", _n_out(5376)),
    3: Workload(3, 32700, 5376, 16128, "w8a8", _n_out(5376)),
    4: Workload(4, 14850, 7168, 28672, "w8a8", _n_out(7168)),
    5: Workload(5, 8192, 28672, 7168, "w4a4", _n_out(28672)),
}


def workload(cid: int) -> Workload:
    return WORKLOADS[cid]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round FP32 to BF16 (nearest-even) with torch's CPU cast; return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to FP32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def outlier_columns(w: Workload) -> np.ndarray:
    return np.sort(_rng(4000 + w.cid).choice(w.K, size=w.n_outliers, replace=False))


CHUNK_ROWS = 2048


def iter_x(w: Workload, rows: int | None = None, chunk_rows: int = CHUNK_ROWS):
    """Yield (r0, r1, bits) for consecutive row chunks of the BF16 activations.

    The values are exactly those of one standard_normal draw of shape [M, K]
    from the seeded generator (the generator is consumed in row order), so
    chunking changes nothing.  ``rows`` stops after that many leading rows.
    ``bits`` is a reused uint16 buffer: consume it before the next step."""
    import torch
    M = w.M if rows is None else min(rows, w.M)
    g = _rng(1000 + w.cid)
    cols = outlier_columns(w)
    cr = max(1, min(chunk_rows, M))
    buf = np.empty((cr, w.K), np.float32)
    tb = torch.empty((cr, w.K), dtype=torch.bfloat16)
    for r0 in range(0, M, cr):
        r1 = min(M, r0 + cr)
        b = buf[: r1 - r0]
        g.standard_normal(out=b, dtype=np.float32)
        b[:, cols] *= np.float32(20.0)
        t = tb[: r1 - r0]
        t.copy_(torch.from_numpy(b))          # round to nearest-even
        yield r0, r1, t.view(torch.int16).numpy().view(np.uint16)


def make_x(w: Workload, rows: int | None = None) -> np.ndarray:
    """BF16 activations [M, K] (or the leading ``rows`` rows) as uint16 bit patterns."""
    M = w.M if rows is None else min(rows, w.M)
    out = np.empty((M, w.K), np.uint16)
    for r0, r1, bits in iter_x(w, rows):
        out[r0:r1] = bits
    return out


def iter_w(w: Workload, chunk_rows: int = CHUNK_ROWS):
    """Yield (r0, r1, fp32 chunk) of the weights [N, K] ~ N(0, 0.02) (reused buffer)."""
    g = _rng(2000 + w.cid)
    cr = min(chunk_rows, w.N)
    buf = np.empty((cr, w.K), np.float32)
    for r0 in range(0, w.N, cr):
        r1 = min(w.N, r0 + cr)
        b = buf[: r1 - r0]
        g.standard_normal(out=b, dtype=np.float32)
        b *= np.float32(0.02)
        yield r0, r1, b


def make_w(w: Workload) -> np.ndarray:
    """FP32 weights [N, K] ~ N(0, 0.02)."""
    out = np.empty((w.N, w.K), np.float32)
    for r0, r1, b in iter_w(w):
        out[r0:r1] = b
    return out


def make_bias(w: Workload) -> np.ndarray:
    """BF16 bias [N] as uint16 bit patterns, ~ N(0, 0.1)."""
    g = _rng(3000 + w.cid)
    return f32_to_bf16_bits(g.standard_normal(w.N, dtype=np.float32) * np.float32(0.1))


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """Generic seeded BF16 tensor (uint16 bits), N(0, scale^2)."""
    g = _rng(seed)
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(scale))
