"""A deterministic sweep of shapes drawn from a fixed seed through the
layer's main entry points, against the oracle: the rotated INT8 layer on
K-sliced weights (BF16 within one ulp, and the same bits as the row-major
entry point), the INT8 GEMM's INT32 accumulators (bit for bit) with either
output tile, and the FP6 W4A4 GEMM's exact sums.  The shapes mix ragged M
and N (tile and column tails, N % 8 != 0) with K from one rotation block to
several LDS rings."""
import numpy as np
import pytest

from gpu_util import assert_bf16_within_1ulp, bf16_bits, host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import quantized_diffusion_amd as q
    q.lib()
    return q


def _shapes(seed, n, kstep, kmax):
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        M = int(g.integers(1, 700))
        N = int(g.integers(1, 1300))
        K = int(g.integers(1, kmax // kstep + 1)) * kstep
        out.append((M, N, K))
    return out


LINEAR_SHAPES = _shapes(20240, 10, 256, 3072)
GEMM_SHAPES = _shapes(20241, 10, 64, 2048)
FP6_SHAPES = _shapes(20242, 8, 128, 2048)


@pytest.mark.parametrize("i", range(len(LINEAR_SHAPES)))
def test_sweep_int8_linear_sliced(qd, O, i):
    import torch
    from synth import f32_to_bf16_bits
    M, N, K = LINEAR_SHAPES[i]
    tiles = 1 + i % 2
    say(f"sweep int8_linear_sliced M={M} N={N} K={K} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(7000 + i))
    x = f32_to_bf16_bits(g.standard_normal((M, K), dtype=np.float32) * np.float32(1 + i))
    W = (g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    b = f32_to_bf16_bits((g.standard_normal(N, dtype=np.float32) * np.float32(0.1)).astype(np.float32))
    wqo, swo = O.prepare_weights(W)
    wq, sw, bd, xd = to_dev(wqo), to_dev(swo), to_dev_bf16(b), to_dev_bf16(x)
    qd.set_gemm_tiles(tiles)
    try:
        y = qd.int8_linear_sliced(xd, qd.slice_weights(wq), sw, bd)
        y_rm = qd.int8_linear(xd, wq, sw, bd)
    finally:
        qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)
    assert torch.equal(y, y_rm)
    assert_bf16_within_1ulp(bf16_bits(y), O.linear(x, wqo, swo, b), f"sweep linear {M}x{N}x{K}")


@pytest.mark.parametrize("i", range(len(GEMM_SHAPES)))
def test_sweep_gemm_i32(qd, O, i):
    M, N, K = GEMM_SHAPES[i]
    g = np.random.Generator(np.random.PCG64(7100 + i))
    a = g.integers(-128, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    want = O.gemm_i32(a, w)
    for tiles in (1, 2):
        say(f"sweep gemm i32 M={M} N={N} K={K} tiles={tiles}")
        qd.set_gemm_tiles(tiles)
        try:
            acc = qd.int8_gemm_i32(to_dev(a), to_dev(w))
            acc_sl = qd.int8_gemm_i32_sliced(to_dev(a), qd.slice_weights(to_dev(w)))
        finally:
            qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)
        assert np.array_equal(host(acc), want), (M, N, K, tiles)
        assert np.array_equal(host(acc_sl), want), (M, N, K, tiles, "sliced")


@pytest.mark.parametrize("i", range(len(FP6_SHAPES)))
def test_sweep_fp6_gemm(qd, O, i):
    M, N, K = FP6_SHAPES[i]
    say(f"sweep fp6 gemm M={M} N={N} K={K}")
    g = np.random.Generator(np.random.PCG64(7200 + i))
    a = g.integers(-7, 8, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-7, 8, (N, K), dtype=np.int64).astype(np.int8)
    want = O.gemm_i32(a, w)
    a6, w6 = qd.pack_fp6(to_dev(a)), qd.pack_fp6(to_dev(w))
    assert np.array_equal(host(qd.fp6_gemm_i32(a6, w6, K)), want), (M, N, K)
    assert np.array_equal(host(qd.fp6_gemm_i32_sliced(a6, qd.fp6_slice_weights(w6, K))), want), (M, N, K, "sliced")
