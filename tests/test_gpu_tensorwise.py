"""GPU parity of the tensor-wise row: quantize_int8_tensorwise (one scale for
the whole tensor) and the GEMM with per-tensor scales, through the C ABI,
against the oracle.  Codes and the scale bit for bit; BF16 outputs within one
BF16 ulp (expected identical; the differing count is printed)."""
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


def _x(shape, seed, scale=1.0, outliers=0):
    from synth import f32_to_bf16_bits
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    if outliers:
        x[:, g.choice(shape[1], size=outliers, replace=False)] *= 20
    return f32_to_bf16_bits(x)


def _check_tw(qd, O, x_dev, x_host, dtype, what):
    q, s = qd.quantize_int8_tensorwise(x_dev)
    qo, so = O.quantize_tensorwise(x_host, dtype)
    assert host(s).view(np.uint32)[0] == so.view(np.uint32)[0], (what, host(s)[0], so[0])
    qq = host(q)
    bad = np.flatnonzero(qq.reshape(-1) != qo.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} codes differ, first at flat index {int(bad[0])}"


@pytest.mark.parametrize("M,K", [(1, 16), (3, 48), (257, 528), (64, 5376), (1500, 1024), (2, 65536)])
def test_tensorwise_bf16(qd, O, M, K):
    say(f"tensorwise bf16 M={M} K={K}")
    x = _x((M, K), seed=500 + M + K, outliers=max(1, K // 100))
    _check_tw(qd, O, to_dev_bf16(x), x, "bf16", f"M={M} K={K}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("M,K", [(5, 32), (300, 1040)])
def test_tensorwise_other_dtypes(qd, O, dtype, M, K):
    say(f"tensorwise {dtype} M={M} K={K}")
    g = np.random.Generator(np.random.PCG64(600 + M))
    x = (g.standard_normal((M, K)) * 0.7).astype(np.float32 if dtype == "f32" else np.float16)
    _check_tw(qd, O, to_dev(x), x, dtype, f"{dtype} M={M} K={K}")


def test_tensorwise_max_in_last_row_and_near_ties(qd, O):
    """The tensor maximum sits in the last row (several rows per workgroup, so
    it must travel through the partial maxima); every other value is placed
    next to a half-integer multiple of the global scale."""
    say("tensorwise near ties, M=3000 K=64")
    M, K = 3000, 64
    g = np.random.Generator(np.random.PCG64(610))
    amax = np.float32(45.0)
    s = np.float32(amax / np.float32(127))
    k = g.integers(-126, 126, size=(M, K))
    x = ((k + 0.5) * np.float64(s)).astype(np.float32)
    step = g.choice([-1, 0, 1], size=(M, K))
    x = np.where(step > 0, np.nextafter(x, np.float32(np.inf)), np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), x))
    x = x.astype(np.float32)
    x[M - 1, K - 1] = amax
    _check_tw(qd, O, to_dev(x), x, "f32", "near ties")


def test_tensorwise_degenerate(qd, O):
    say("tensorwise zero / subnormal / single spike")
    z = np.zeros((40, 256), np.uint16)
    _check_tw(qd, O, to_dev_bf16(z), z, "bf16", "zero")
    g = np.random.Generator(np.random.PCG64(620))
    sub = (g.integers(1, 0x80, (7, 48)) | (g.integers(0, 2, (7, 48)) << 15)).astype(np.uint16)   # BF16 subnormals
    _check_tw(qd, O, to_dev_bf16(sub), sub, "bf16", "subnormal")
    spike = np.zeros((1025, 32), np.uint16)
    spike[517, 9] = 0xC2C8                                                                   # -100
    _check_tw(qd, O, to_dev_bf16(spike), spike, "bf16", "spike")


def test_tensorwise_strided_and_reused_workspace(qd, O):
    import torch
    say("tensorwise strided rows, workspace reused by a smaller call")
    x = _x((100, 1024), seed=630)
    xd = to_dev_bf16(x)[:, :768]                     # row stride 1024, K = 768
    ws = torch.empty(qd.tensorwise_workspace_size(), dtype=torch.uint8, device="cuda")
    q, s = qd.quantize_int8_tensorwise(xd, workspace=ws)
    qo, so = O.quantize_tensorwise(np.ascontiguousarray(x[:, :768]), "bf16")
    assert np.array_equal(host(q), qo) and host(s)[0] == so[0]
    x2 = _x((9, 64), seed=631, scale=3.0)
    q2, s2 = qd.quantize_int8_tensorwise(to_dev_bf16(x2), workspace=ws)
    qo2, so2 = O.quantize_tensorwise(x2, "bf16")
    assert np.array_equal(host(q2), qo2) and host(s2)[0] == so2[0]


@pytest.mark.parametrize("a_tensor,w_tensor", [(True, True), (True, False), (False, True), (False, False)])
@pytest.mark.parametrize("M,N,K", [(257, 1000, 5376), (70, 264, 528)])
@pytest.mark.parametrize("tiles", [1, 2])
def test_scaled_mm_ex(qd, O, a_tensor, w_tensor, M, N, K, tiles):
    say(f"scaled_mm_ex M={M} N={N} K={K} a_tensor={a_tensor} w_tensor={w_tensor} tiles={tiles}")
    qd.set_gemm_tiles(tiles)
    g = np.random.Generator(np.random.PCG64(M * 3 + N + K + 2 * a_tensor + w_tensor))
    a = g.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    sx = (g.uniform(0.5, 2.0, 1 if a_tensor else M) * 2.0 ** -7).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, 1 if w_tensor else N) * 2.0 ** -12).astype(np.float32)
    from synth import random_bf16
    b = random_bf16(N, seed=K + 1, scale=0.1)
    y = qd.int8_scaled_mm_ex(to_dev(a), to_dev(sx), to_dev(w), to_dev(sw), to_dev_bf16(b))
    qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)
    yo = O.epilogue(O.gemm_i32(a, w), np.broadcast_to(sx, (M,)), np.broadcast_to(sw, (N,)), b)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "scaled_mm_ex")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


def test_tensorwise_linear_pipeline(qd, O):
    """Tensor-wise activation codes feeding the per-tensor-activation GEMM."""
    say("tensorwise pipeline M=300 N=520 K=1024")
    M, N, K = 300, 520, 1024
    x = _x((M, K), seed=640, outliers=10)
    g = np.random.Generator(np.random.PCG64(641))
    wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, sw = O.quantize_rowwise(wf, "f32", 0)
    from synth import random_bf16
    b = random_bf16(N, seed=642, scale=0.1)
    aq, sa = qd.quantize_int8_tensorwise(to_dev_bf16(x))
    y = qd.int8_scaled_mm_ex(aq, sa, to_dev(wq), to_dev(sw), to_dev_bf16(b))
    aqo, sao = O.quantize_tensorwise(x, "bf16")
    yo = O.epilogue(O.gemm_i32(aqo, wq), np.broadcast_to(sao, (M,)), sw, b)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "tensorwise pipeline")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


def test_tensorwise_full_size(qd, O):
    """The activation tensor of the M8193/K5376/N16128 workload, every code."""
    from synth import make_x, workload
    w = workload(2)
    say(f"tensorwise full size {w.name}")
    x = make_x(w)
    _check_tw(qd, O, to_dev_bf16(x), x, "bf16", w.name)
