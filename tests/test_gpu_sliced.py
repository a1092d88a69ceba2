"""K-sliced INT8 weights: the re-layout against numpy's reshape, and the GEMM
and the whole layer on sliced weights against the oracle (INT32 bit for bit,
BF16 within one ulp) and against the row-major entry points (bit for bit:
the same kernels with other copy addresses)."""
import numpy as np
import pytest

from fp6_format import assert_fp6_codes, unslice96
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


@pytest.fixture(params=[1, 2], ids=["tiles256x256", "tiles256x384"])
def tiles(request, qd):
    qd.set_gemm_tiles(request.param)
    yield request.param
    qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)


def _codes(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(-128, 128, shape, dtype=np.int64).astype(np.int8)


@pytest.mark.parametrize("N,K,pad", [(1, 64, 0), (8, 128, 16), (255, 320, 0), (384, 5376, 64), (1000, 1024, 0)])
def test_slice_weights_layout(qd, N, K, pad):
    """Element [u, n, j] of the sliced copy is wq[n, 64 u + j] (also from a strided wq)."""
    import torch
    say(f"slice_weights N={N} K={K} pad={pad}")
    w = _codes((N, K + pad), 10 + N + K)
    wd = to_dev(w)[:, :K]
    ws = qd.slice_weights(wd)
    assert ws.shape == (K // 64, N, 64) and ws.dtype == torch.int8
    ref = np.ascontiguousarray(w[:, :K].reshape(N, K // 64, 64).transpose(1, 0, 2))
    assert np.array_equal(host(ws), ref)


SHAPES = [(1, 1, 64), (256, 256, 64), (257, 255, 128), (70, 130, 128), (300, 520, 512),
          (513, 1000, 5376), (64, 4100, 1024), (300, 520, 256), (257, 264, 320), (300, 520, 448)]


def _slice_np(a):
    """[R, K] -> the K-sliced layout [K / 64, R, 64] (numpy reshape)."""
    R, K = a.shape
    return np.ascontiguousarray(a.reshape(R, K // 64, 64).transpose(1, 0, 2))


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_sliced_gemm_i32_exact(qd, O, tiles, M, N, K):
    """K-sliced weights with row-major and with K-sliced activation codes."""
    say(f"sliced gemm i32 M={M} N={N} K={K} tiles={tiles}")
    a = _codes((M, K), M * 7 + N * 3 + K)
    w = _codes((N, K), M * 5 + N * 11 + K)
    wd = to_dev(w)
    wsl = qd.slice_weights(wd)
    ref = O.gemm_i32(a, w)
    assert np.array_equal(host(qd.int8_gemm_i32_sliced(to_dev(a), wsl)), ref)
    assert np.array_equal(host(qd.int8_gemm_i32_sliced(to_dev(_slice_np(a)), wsl)), ref)
    assert np.array_equal(host(qd.int8_gemm_i32(to_dev(a), wd)), ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("M,K", [(1, 256), (3, 512), (63, 768), (257, 5376), (130, 7168), (1000, 1024),
                                 (7, 28672)])
def test_quantize_sliced(qd, O, dtype, M, K):
    """The rotating quantizer writing K-sliced codes: the oracle's codes re-laid out, same scales."""
    say(f"sliced rotquant {dtype} M={M} K={K}")
    g = np.random.Generator(np.random.PCG64(40 + M + K))
    xf = g.standard_normal((M, K), dtype=np.float32)
    if dtype == "bf16":
        from synth import f32_to_bf16_bits
        x = f32_to_bf16_bits(xf)
        xd = to_dev_bf16(x)
    else:
        x = xf if dtype == "f32" else xf.astype(np.float16)
        xd = to_dev(x)
    q, s = qd.quantize_and_rotate_rowwise_sliced(xd)
    qo, so = O.quantize_rowwise(x, dtype, 256)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), _slice_np(qo))


@pytest.mark.parametrize("act", [1, 2, 3, 4])
def test_quantize_sliced_act(qd, O, act):
    from synth import f32_to_bf16_bits
    say(f"sliced rotquant act={act}")
    g = np.random.Generator(np.random.PCG64(70 + act))
    x = f32_to_bf16_bits(g.standard_normal((77, 1280), dtype=np.float32) * 3)
    q, s = qd.quantize_and_rotate_rowwise_sliced(to_dev_bf16(x), input_act=act)
    qo, so = O.quantize_rowwise(x, "bf16", 256, act=act)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), _slice_np(qo))


def test_sliced_gemm_i32_extremes(qd, O, tiles):
    say(f"sliced gemm i32 extremes tiles={tiles}")
    K = 5376
    a = np.full((300, K), 127, np.int8)
    a[1::2] = -127
    w = np.full((260, K), 127, np.int8)
    w[::3] = -128
    acc = qd.int8_gemm_i32_sliced(to_dev(a), qd.slice_weights(to_dev(w)))
    assert np.array_equal(host(acc), O.gemm_i32(a, w))


@pytest.mark.parametrize("M,N,K,with_bias", [(256, 512, 512, True), (257, 264, 5376, True),
                                              (77, 1000, 768, False), (1, 8, 64, True)])
def test_sliced_scaled_mm(qd, O, tiles, M, N, K, with_bias):
    import torch
    say(f"sliced scaled_mm M={M} N={N} K={K} bias={with_bias} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(M + N + K))
    a = _codes((M, K), 3 * M + K)
    w = _codes((N, K), 5 * N + K)
    sx = (g.random(M, dtype=np.float32) * 1e-3).astype(np.float32)
    sw = (g.random(N, dtype=np.float32) * 1e-3).astype(np.float32)
    b = (g.standard_normal(N, dtype=np.float32) * 0.1).astype(np.float32) if with_bias else None
    from synth import f32_to_bf16_bits
    bb = f32_to_bf16_bits(b) if with_bias else None
    bd = to_dev_bf16(bb) if with_bias else None
    wd = to_dev(w)
    wsl = qd.slice_weights(wd)
    y = qd.int8_scaled_mm_sliced(to_dev(a), to_dev(sx), wsl, to_dev(sw), bd)
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, bb)
    assert_bf16_within_1ulp(bf16_bits(y), yo, "scaled_mm_sliced")
    y_rm = qd.int8_scaled_mm(to_dev(a), to_dev(sx), wd, to_dev(sw), bd)
    assert torch.equal(y, y_rm)
    if K % 64 == 0:
        y_as = qd.int8_scaled_mm_sliced(to_dev(_slice_np(a)), to_dev(sx), wsl, to_dev(sw), bd)
        assert torch.equal(y_as, y_rm)


@pytest.mark.parametrize("act", [0, 1, 3])
@pytest.mark.parametrize("M,rotate", [(1, 256), (255, 256), (300, 256), (77, 0)])
def test_int8_linear_sliced(qd, O, tiles, act, M, rotate):
    """The whole layer on sliced weights: oracle within one ulp, and the same
    bits as int8_linear_act on the row-major codes."""
    import torch
    from synth import make_bias, make_w, workload
    say(f"int8_linear_sliced M={M} act={act} rotate={rotate} tiles={tiles}")
    w = workload(1)
    W, b = make_w(w), make_bias(w)
    g = np.random.Generator(np.random.PCG64(900 + M + act))
    from synth import f32_to_bf16_bits
    x = f32_to_bf16_bits(g.standard_normal((M, w.K), dtype=np.float32))
    wqo, swo = O.prepare_weights(W, block=rotate)
    wq = to_dev(wqo)
    xd, bd = to_dev_bf16(x), to_dev_bf16(b)
    y = qd.int8_linear_sliced(xd, qd.slice_weights(wq), to_dev(swo), bd, input_act=act, rotate_block=rotate)
    y_rm = qd.int8_linear_act(xd, wq, to_dev(swo), bd, input_act=act, rotate_block=rotate)
    assert torch.equal(y, y_rm)
    yo = O.linear(x, wqo, swo, b, block=rotate, act=act)
    assert_bf16_within_1ulp(bf16_bits(y), yo, "int8_linear_sliced")


@pytest.mark.parametrize("M,N,K", [(300, 7, 512), (257, 259, 1024), (513, 1001, 5376), (70, 1003, 256)])
def test_sliced_column_tail(qd, O, tiles, M, N, K):
    """N % 8 in {1, 3, 7} on the K-sliced entry points: int8_scaled_mm_sliced
    (row-major and K-sliced activation codes) and int8_linear_sliced, element
    by element against the oracle; the padding of the output rows untouched."""
    import torch
    from synth import f32_to_bf16_bits
    say(f"sliced column tail M={M} N={N} K={K} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(4 * M + N + K))
    a = _codes((M, K), 9 * M + K)
    w = _codes((N, K), 13 * N + K)
    sx = (g.random(M, dtype=np.float32) * 1e-3).astype(np.float32)
    sw = (g.random(N, dtype=np.float32) * 1e-3).astype(np.float32)
    bb = f32_to_bf16_bits((g.standard_normal(N, dtype=np.float32) * 0.1).astype(np.float32))
    bd = to_dev_bf16(bb)
    wsl = qd.slice_weights(to_dev(w))
    ldy = (N + 7) // 8 * 8
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, bb)
    for a_dev, what in ((to_dev(a), "row-major codes"), (to_dev(_slice_np(a)), "K-sliced codes")):
        buf = torch.full((M, ldy), 3.0, dtype=torch.bfloat16, device="cuda")
        y = qd.int8_scaled_mm_sliced(a_dev, to_dev(sx), wsl, to_dev(sw), bd, out=buf[:, :N])
        assert_bf16_within_1ulp(bf16_bits(y), yo, f"scaled_mm_sliced column tail, {what}")
        assert torch.all(buf[:, N:] == 3.0), "the row padding past N was written"
    # the whole layer (rotated, with bias) on N % 8 != 0
    x = f32_to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    W = (g.standard_normal((N, K), dtype=np.float32) * 0.02).astype(np.float32)
    wqo, swo = O.prepare_weights(W)
    buf = torch.full((M, ldy), 3.0, dtype=torch.bfloat16, device="cuda")
    y = qd.int8_linear_sliced(to_dev_bf16(x), qd.slice_weights(to_dev(wqo)), to_dev(swo), bd, out=buf[:, :N])
    assert_bf16_within_1ulp(bf16_bits(y), O.linear(x, wqo, swo, bb), "int8_linear_sliced column tail")
    assert torch.all(buf[:, N:] == 3.0), "the row padding past N was written"


def test_int8_linear_sliced_full_size(qd, O):
    """The M32700/K5376/N16128 workload in the launch configuration the
    benchmark times: the same bits as int8_linear on row-major weights, and
    sampled outputs against the oracle."""
    import torch
    from synth import iter_w, iter_x, make_bias, workload
    w = workload(3)
    M, K, N = w.M, w.K, w.N
    dev = torch.device("cuda:0")
    say(f"sliced full-size {w.name}: inputs")
    x_host = np.empty((M, K), np.uint16)
    xd = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    for r0, r1, bits in iter_x(w):
        x_host[r0:r1] = bits
        xd[r0:r1].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    W = np.empty((N, K), np.float32)
    Wd = torch.empty((N, K), dtype=torch.float32, device=dev)
    for r0, r1, chunk in iter_w(w):
        W[r0:r1] = chunk
        Wd[r0:r1].copy_(torch.from_numpy(chunk))
    b = make_bias(w)
    bd = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev)
    wq, sw = qd.prepare_weights(Wd)
    del Wd
    wsl = qd.slice_weights(wq)
    ws = torch.empty(qd.workspace_size(M, K), dtype=torch.uint8, device=dev)
    say("  int8_linear_sliced and int8_linear")
    y = qd.int8_linear_sliced(xd, wsl, sw, bd, workspace=ws)
    y_rm = qd.int8_linear(xd, wq, sw, bd, 256, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, y_rm)
    del y_rm
    say("  sampled outputs against the oracle")
    wqo, swo = O.prepare_weights(W)
    del W
    qo, so = O.quantize_rowwise(x_host, "bf16", 256)
    g = np.random.Generator(np.random.PCG64(9300))
    rows = np.concatenate([g.integers(0, M, 4000), np.full(N, M - 1)])
    cols = np.concatenate([g.integers(0, N, 4000), np.arange(N)])
    yo, _ = O.linear_points(qo, so, rows, wqo, swo, b, cols)
    yg = bf16_bits(y[torch.from_numpy(rows).to(dev), torch.from_numpy(cols).to(dev)])
    assert_bf16_within_1ulp(yg, yo, "sliced full size")


# ----------------------------------------------------------- K-sliced FP6

def _slice96(b):
    """Row-major FP6 bytes [R, 3K/4] -> the K-sliced layout [K / 128, R, 96]."""
    R, B = b.shape
    return np.ascontiguousarray(b.reshape(R, B // 96, 96).transpose(1, 0, 2))


def _int4(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(-7, 8, shape, dtype=np.int64).astype(np.int8)


@pytest.mark.parametrize("N,K", [(1, 128), (255, 384), (384, 5376), (1000, 1024)])
def test_fp6_slice_weights_layout(qd, O, N, K):
    say(f"fp6 slice N={N} K={K}")
    w4 = _int4((N, K), 300 + N + K)
    w6 = qd.pack_fp6(to_dev(w4))
    ws = qd.fp6_slice_weights(w6, K)
    assert np.array_equal(host(ws), _slice96(host(w6)))
    assert_fp6_codes(unslice96(host(ws), N), w4, "fp6 sliced weights")


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (257, 255, 256), (70, 130, 384), (300, 520, 1024), (513, 1000, 5376),
                                   (300, 520, 640), (257, 264, 512)])
def test_fp6_sliced_gemm_exact(qd, O, M, N, K):
    say(f"fp6 sliced gemm M={M} N={N} K={K}")
    a4, w4 = _int4((M, K), 7 * M + K), _int4((N, K), 11 * N + K)
    a6 = qd.pack_fp6(to_dev(a4))
    w6s = qd.fp6_slice_weights(qd.pack_fp6(to_dev(w4)), K)
    ref = O.gemm_i32(a4, w4)
    assert np.array_equal(host(qd.fp6_gemm_i32_sliced(a6, w6s)), ref)
    assert np.array_equal(host(qd.fp6_gemm_i32_sliced(to_dev(_slice96(host(a6))), w6s)), ref)


def test_fp6_sliced_gemm_extremes(qd, O):
    """|sum| = 49 K at K = 28672: the FP32 accumulators stay exact on the sliced path."""
    K = 28672
    a4 = np.full((300, K), 7, np.int8)
    a4[1::2] = -7
    w4 = np.full((260, K), 7, np.int8)
    w4[::3] = -7
    w6s = qd.fp6_slice_weights(qd.pack_fp6(to_dev(w4)), K)
    acc = qd.fp6_gemm_i32_sliced(qd.pack_fp6(to_dev(a4)), w6s)
    assert np.array_equal(host(acc), O.gemm_i32(a4, w4))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,K", [(1, 256), (63, 768), (257, 5376), (5, 28672)])
def test_quantize_fp6_sliced(qd, O, dtype, M, K):
    say(f"fp6 sliced quantizer {dtype} M={M} K={K}")
    g = np.random.Generator(np.random.PCG64(500 + M + K))
    xf = g.standard_normal((M, K), dtype=np.float32)
    if dtype == "bf16":
        from synth import f32_to_bf16_bits
        x = f32_to_bf16_bits(xf)
        xd = to_dev_bf16(x)
    else:
        x = xf.astype(np.float16)
        xd = to_dev(x)
    q6, s = qd.quantize_and_rotate_rowwise_fp6_sliced(xd)
    qo, so = O.quantize_rowwise(x, dtype, 256, qmax=7)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert_fp6_codes(unslice96(host(q6), M), qo, "fp6 sliced quantizer")


@pytest.mark.parametrize("M,K,N", [(1, 256, 8), (255, 512, 264), (300, 1024, 520), (257, 5376, 1000)])
def test_convrot_w4a4_linear_fp6_sliced(qd, O, M, K, N):
    """The FP6 layer on K-sliced operands: the same bits as the row-major FP6
    layer, and the oracle's W4A4 layer within one ulp."""
    import torch
    from synth import f32_to_bf16_bits
    say(f"w4a4 fp6 sliced M={M} K={K} N={N}")
    g = np.random.Generator(np.random.PCG64(800 + M + K + N))
    x = f32_to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    W = (g.standard_normal((N, K), dtype=np.float32) * 0.02).astype(np.float32)
    b = f32_to_bf16_bits((g.standard_normal(N, dtype=np.float32) * 0.1).astype(np.float32))
    w6, sw = qd.prepare_weights_w4a4_fp6(to_dev(W))
    xd, bd = to_dev_bf16(x), to_dev_bf16(b)
    y = qd.convrot_w4a4_linear_fp6_sliced(xd, qd.fp6_slice_weights(w6, K), sw, bd)
    y_rm = qd.convrot_w4a4_linear_fp6(xd, w6, sw, bd)
    assert torch.equal(y, y_rm)
    wqo, swo = O.prepare_weights(W, qmax=7)
    assert_bf16_within_1ulp(bf16_bits(y), O.linear(x, wqo, swo, b, qmax=7), "w4a4 fp6 sliced")


def test_w4a4_fp6_sliced_full_size(qd):
    """The M8192/K28672/N7168 W4A4 workload as the benchmark times it: the
    same bits as the row-major FP6 layer (whose full-size parity with the
    oracle is tested in test_gpu_fp6)."""
    import torch
    from synth import iter_w, iter_x, make_bias, workload
    w = workload(5)
    M, K, N = w.M, w.K, w.N
    dev = torch.device("cuda:0")
    say(f"fp6 sliced full-size {w.name}")
    xd = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    for r0, r1, bits in iter_x(w):
        xd[r0:r1].copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))
    Wd = torch.empty((N, K), dtype=torch.float32, device=dev)
    for r0, r1, chunk in iter_w(w):
        Wd[r0:r1].copy_(torch.from_numpy(chunk))
    bd = torch.from_numpy(make_bias(w).view(np.int16)).view(torch.bfloat16).to(dev)
    w6, sw = qd.prepare_weights_w4a4_fp6(Wd)
    del Wd
    y = qd.convrot_w4a4_linear_fp6_sliced(xd, qd.fp6_slice_weights(w6, K), sw, bd)
    y_rm = qd.convrot_w4a4_linear_fp6(xd, w6, sw, bd)
    torch.cuda.synchronize()
    assert torch.equal(y, y_rm)


def test_int8_linear_sliced_strided_and_degenerate(qd, O):
    """x with a row stride above K, a zero row and a row of one spike, no bias,
    a reused workspace: the same bits as int8_linear, and the oracle."""
    import torch
    from synth import f32_to_bf16_bits, make_w, workload
    w = workload(1)
    W = make_w(w)
    g = np.random.Generator(np.random.PCG64(4242))
    M, K = 65, w.K
    xf = g.standard_normal((M, K + 64), dtype=np.float32)
    xf[3] = 0.0
    xf[7] = 0.0
    xf[7, 100] = 5.0
    x = f32_to_bf16_bits(xf)
    xd = to_dev_bf16(x)[:, :K]
    wqo, swo = O.prepare_weights(W)
    wq = to_dev(wqo)
    ws = torch.empty(qd.workspace_size(M, K), dtype=torch.uint8, device=xd.device)
    y = qd.int8_linear_sliced(xd, qd.slice_weights(wq), to_dev(swo), None, workspace=ws)
    y_rm = qd.int8_linear(xd, wq, to_dev(swo), None, 256, ws)
    assert torch.equal(y, y_rm)
    assert_bf16_within_1ulp(bf16_bits(y), O.linear(np.ascontiguousarray(x[:, :K]), wqo, swo, None), "strided")
    assert not bf16_bits(y)[3].any()    # zero row, no bias: +0 everywhere
