"""GPU parity: the HIP library (through its C ABI) against the oracle on the
same seeded inputs.  Codes, row scales and INT32 accumulators must match bit
for bit; BF16 outputs within one BF16 ulp of the oracle (the expected result
is bit-identical, and the count of differing values is printed)."""
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
    from synth import random_bf16
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    if outliers:
        cols = g.choice(shape[1], size=outliers, replace=False)
        x[:, cols] *= 20
    from synth import f32_to_bf16_bits
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------------- quantizers

@pytest.mark.parametrize("M,K", [(1, 256), (3, 512), (63, 768), (256, 512), (257, 5376), (130, 7168),
                                 (5, 28672), (2, 65536), (1000, 1024)])
def test_rotquant_bf16(qd, O, M, K):
    say(f"rotquant bf16 M={M} K={K}")
    x = _x((M, K), seed=100 + M + K, outliers=max(1, K // 100))
    q, s = qd.quantize_and_rotate_rowwise(to_dev_bf16(x))
    qo, so = O.quantize_rowwise(x, "bf16", 256)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("M,K", [(7, 256), (129, 1280), (33, 5376)])
def test_rotquant_other_dtypes(qd, O, dtype, M, K):
    import torch
    say(f"rotquant {dtype} M={M} K={K}")
    g = np.random.Generator(np.random.PCG64(200 + M))
    x = (g.standard_normal((M, K)) * 0.5).astype(np.float32 if dtype == "f32" else np.float16)
    q, s = qd.quantize_and_rotate_rowwise(to_dev(x))
    qo, so = O.quantize_rowwise(x, dtype, 256)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


def test_rotquant_near_ties_and_degenerate_rows(qd, O):
    """Rows whose rotated values sit next to half-integer multiples of the scale
    (the exact-division fallback), tiny-scale rows (the all-exact path), zero
    rows, subnormal rows and single spikes."""
    from exact import sylvester
    say("rotquant near-ties / degenerate rows")
    H = sylvester(256).astype(np.float64) / 16.0
    g = np.random.Generator(np.random.PCG64(300))
    rows = []
    for t in range(24):
        v = (g.integers(-126, 126, 512) + 0.5).astype(np.float64)
        v[0] = 127.0
        v *= 2.0 ** g.integers(-8, 8)
        x = np.concatenate([H @ v[:256], H @ v[256:]])          # rotate(x) ~ v
        rows.append(x.astype(np.float32))
    rows.append(np.zeros(512, np.float32))
    rows.append((g.standard_normal(512) * 1e-36).astype(np.float32))      # scale < 2^-100
    rows.append((g.standard_normal(512) * 1e-30).astype(np.float32))
    sub = np.zeros(512, np.float32)
    sub[::7] = np.float32(1e-45) * g.integers(1, 50, sub[::7].size)
    rows.append(sub)                                                       # subnormal inputs
    spike = np.zeros(512, np.float32)
    spike[300] = -3.0
    rows.append(spike)
    x = np.stack(rows)
    q, s = qd.quantize_and_rotate_rowwise(to_dev(x))
    qo, so = O.quantize_rowwise(x, "f32", 256)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)
    # the same through the INT4 quantizer
    q4, s4 = qd.quantize_and_rotate_rowwise_int4(to_dev(x))
    qo4, so4 = O.quantize_rowwise(x, "f32", 256, qmax=7)
    assert np.array_equal(host(s4).view(np.uint32), so4.view(np.uint32))
    assert np.array_equal(host(q4), qo4)


@pytest.mark.parametrize("M,K", [(1, 16), (5, 48), (64, 272), (257, 5376), (3, 4096)])
def test_quantize_int8_rowwise(qd, O, M, K):
    say(f"quantize_int8_rowwise M={M} K={K}")
    x = _x((M, K), seed=400 + K, outliers=1)
    q, s = qd.quantize_int8_rowwise(to_dev_bf16(x))
    qo, so = O.quantize_rowwise(x, "bf16", 0)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


@pytest.mark.parametrize("M,K", [(9, 512), (300, 28672)])
def test_rotquant_int4(qd, O, M, K):
    say(f"rotquant int4 M={M} K={K}")
    x = _x((M, K), seed=500 + M, outliers=K // 100)
    q, s = qd.quantize_and_rotate_rowwise_int4(to_dev_bf16(x))
    qo, so = O.quantize_rowwise(x, "bf16", 256, qmax=7)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


def test_quantize_strided_rows(qd, O):
    """Row strides larger than K on input and output."""
    import torch
    say("rotquant strided")
    x = _x((40, 1024), seed=600)
    xd = to_dev_bf16(x)[:, :768]
    qbuf = torch.zeros((40, 800), dtype=torch.int8, device="cuda")
    q, s = qd.quantize_and_rotate_rowwise(xd, out_q=qbuf[:, :768])
    qo, so = O.quantize_rowwise(np.ascontiguousarray(x[:, :768]), "bf16", 256)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    assert np.all(host(qbuf[:, 768:]) == 0)


# ---------------------------------------------------------------------- GEMM

GEMM_SHAPES = [(1, 1, 16), (1, 1, 64), (256, 256, 64), (257, 255, 80), (70, 130, 128), (300, 520, 512),
               (513, 1000, 5376), (64, 4100, 1024), (1024, 1024, 7168)]


@pytest.fixture(params=[1, 2], ids=["tiles256x256", "tiles256x384"])
def tiles(request, qd):
    """Both INT8 GEMM output tiles on every shape (K % 64 == 0; the general
    kernel otherwise)."""
    qd.set_gemm_tiles(request.param)
    yield request.param
    qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32_exact(qd, O, tiles, M, N, K):
    say(f"gemm i32 M={M} N={N} K={K} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(M * 7 + N * 3 + K))
    a = g.integers(-128, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    acc = qd.int8_gemm_i32(to_dev(a), to_dev(w))
    assert np.array_equal(host(acc), O.gemm_i32(a, w))


@pytest.mark.parametrize("K", [192, 256, 320, 384, 448])
def test_gemm_i32_ring_boundaries(qd, O, tiles, K):
    """K slices around the LDS ring depth (3 to 7 slices of 64): the K loop's
    steady phase (slices with the whole ring after them) and its last slices
    meet at every possible point; INT32 bit for bit, ragged M and N."""
    say(f"gemm i32 ring boundary K={K} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(3 * K + tiles))
    a = g.integers(-128, 128, (300, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-128, 128, (520, K), dtype=np.int64).astype(np.int8)
    assert np.array_equal(host(qd.int8_gemm_i32(to_dev(a), to_dev(w))), O.gemm_i32(a, w))


def test_gemm_i32_largest_stride(qd, O, tiles):
    """Operand rows QD_MAX_LD_GEMM bytes apart (the largest stride accepted:
    a tile's copy offsets reach 383 rows x the stride): INT32 bit for bit."""
    import os
    import re
    import torch
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qdiff.h")
    ld = int(re.search(r"#define QD_MAX_LD_GEMM (\d+)", open(hdr).read()).group(1))
    M, N, K = 300, 520, 256
    say(f"gemm i32 row stride {ld} M={M} N={N} K={K} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(71 + tiles))
    a = g.integers(-128, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-128, 128, (N, K), dtype=np.int64).astype(np.int8)
    ab = torch.zeros((M, ld), dtype=torch.int8, device="cuda")
    wb = torch.zeros((N, ld), dtype=torch.int8, device="cuda")
    ab[:, :K] = to_dev(a)
    wb[:, :K] = to_dev(w)
    acc = qd.int8_gemm_i32(ab[:, :K], wb[:, :K])
    assert np.array_equal(host(acc), O.gemm_i32(a, w))
    del ab, wb


def test_scaled_mm_largest_output_stride(qd, O, tiles):
    """BF16 output rows QD_MAX_LD_GEMM elements apart (the largest output
    stride accepted: the store offsets reach 159 rows x 2 x the stride bytes),
    with whole tiles (first tile row) and a partial one (second tile row):
    within 1 ulp of the oracle, and nothing written between the rows."""
    import os
    import re
    import torch
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qdiff.h")
    ld = int(re.search(r"#define QD_MAX_LD_GEMM (\d+)", open(hdr).read()).group(1))
    M, N, K = 300, 768, 512
    say(f"scaled_mm output row stride {ld} M={M} N={N} K={K} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(73 + tiles))
    a = g.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    sx = (g.uniform(0.5, 2.0, M) * 2.0 ** -7).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, N) * 2.0 ** -12).astype(np.float32)
    from synth import random_bf16
    b = random_bf16(N, seed=74, scale=0.1)
    yb = torch.full((M, ld), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    y = yb[:, :N]
    qd.int8_scaled_mm(to_dev(a), to_dev(sx), to_dev(w), to_dev(sw), to_dev_bf16(b), out=y)
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, b)
    assert_bf16_within_1ulp(bf16_bits(y), yo, "scaled_mm largest output stride")
    gap = yb[:, N:N + 4096].view(torch.int16)
    assert bool((gap == -1).all()), "writes outside the output rows"
    del yb, y


def test_scaled_mm_no_bias_tiny_scales(qd, O, tiles):
    """Without bias, scales so small that the products are FP32 subnormals or
    round to zero: every output bit for bit as the oracle's, the sign of zero
    included (a kernel that added +0 for the missing bias would turn every -0
    into +0)."""
    say(f"scaled_mm no bias, subnormal products tiles={tiles}")
    M, N, K = 300, 776, 512
    g = np.random.Generator(np.random.PCG64(75 + tiles))
    a = g.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    a[::7] = 0        # zero rows: +0 outputs
    a[1::5, ::2] = 1  # small sums of either sign
    # row scales 2^-60, 2^-70, 2^-80 in turn: products from normal through
    # subnormal (FP32 and BF16) to zero
    sx = (g.uniform(0.5, 2.0, M) * 2.0 ** (-60.0 - 10.0 * (np.arange(M) % 3))).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, N) * 2.0 ** -66).astype(np.float32)
    y = qd.int8_scaled_mm(to_dev(a), to_dev(sx), to_dev(w), to_dev(sw), None)
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, None)
    got = bf16_bits(y).reshape(-1)
    want = yo.reshape(-1)
    assert int((want == 0x8000).sum()) > 1000 and int((want == 0).sum()) > 1000
    assert int((((want & 0x7F80) == 0) & ((want & 0x7F) != 0)).sum()) > 1000   # BF16 subnormals
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} outputs differ, first at {bad[0]}: {got[bad[0]]:#06x} vs {want[bad[0]]:#06x}"


@pytest.mark.parametrize("K", [64, 128, 192, 256, 320])
def test_scaled_mm_short_k(qd, O, tiles, K):
    """One to five 64-byte K slices (fewer than the LDS ring holds, so the
    eight-wave kernels never reach their steady loop and the epilogue operand
    loads are issued right after the prologue's copies): BF16 outputs of
    whole and partial tiles within 1 ulp of the oracle."""
    say(f"scaled_mm short K={K} tiles={tiles}")
    from synth import random_bf16
    M, N = 300, 776
    g = np.random.Generator(np.random.PCG64(76 + K + tiles))
    a = g.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    sx = (g.uniform(0.5, 2.0, M) * 2.0 ** -7).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, N) * 2.0 ** -12).astype(np.float32)
    b = random_bf16(N, seed=77 + K, scale=0.1)
    y = qd.int8_scaled_mm(to_dev(a), to_dev(sx), to_dev(w), to_dev(sw), to_dev_bf16(b))
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, b)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, f"scaled_mm K={K}")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


def test_gemm_i32_extremes(qd, O, tiles):
    say(f"gemm i32 extremes tiles={tiles}")
    K = 5376
    a = np.full((300, K), 127, np.int8)
    a[1::2] = -127
    w = np.full((260, K), 127, np.int8)
    w[::3] = -128
    acc = qd.int8_gemm_i32(to_dev(a), to_dev(w))
    assert np.array_equal(host(acc), O.gemm_i32(a, w))


@pytest.mark.parametrize("M,N,K,with_bias", [(256, 512, 512, True), (257, 264, 5376, True),
                                              (77, 1000, 768, False), (1, 8, 16, True)])
def test_scaled_mm_bf16(qd, O, tiles, M, N, K, with_bias):
    say(f"scaled_mm M={M} N={N} K={K} bias={with_bias} tiles={tiles}")
    import torch
    g = np.random.Generator(np.random.PCG64(M + N + K))
    a = g.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    sx = (g.uniform(0.5, 2.0, M) * 2.0 ** -7).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, N) * 2.0 ** -12).astype(np.float32)
    from synth import random_bf16
    b = random_bf16(N, seed=K, scale=0.1) if with_bias else None
    y = qd.int8_scaled_mm(to_dev(a), to_dev(sx), to_dev(w), to_dev(sw), None if b is None else to_dev_bf16(b))
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, b)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "scaled_mm")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


@pytest.mark.parametrize("M,N,K", [(300, 7, 512), (257, 259, 1024), (129, 263, 768), (513, 1001, 5376),
                                   (70, 1003, 320)])
def test_scaled_mm_bf16_column_tail(qd, O, tiles, M, N, K):
    """N % 8 in {1, 3, 7}: the BF16 epilogue's partial 8-column store at the
    right edge, into a row stride padded to 8 whose padding must stay untouched."""
    import torch
    say(f"scaled_mm column tail M={M} N={N} K={K} tiles={tiles}")
    g = np.random.Generator(np.random.PCG64(M + 3 * N + K))
    a = g.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    sx = (g.uniform(0.5, 2.0, M) * 2.0 ** -7).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, N) * 2.0 ** -12).astype(np.float32)
    from synth import random_bf16
    b = random_bf16(N, seed=K + 1, scale=0.1)
    ldy = (N + 7) // 8 * 8
    buf = torch.full((M, ldy), -7.0, dtype=torch.bfloat16, device="cuda")
    y = qd.int8_scaled_mm(to_dev(a), to_dev(sx), to_dev(w), to_dev(sw), to_dev_bf16(b), out=buf[:, :N])
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, b)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "scaled_mm column tail")
    assert torch.all(buf[:, N:] == -7.0), "the row padding past N was written"
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


# ------------------------------------------------------------- whole layer

def test_int8_linear_tiny_config(qd, O):
    """The 256/512/512 workload end to end (bias, outliers, rotation)."""
    from synth import make_bias, make_w, make_x, workload
    say("int8_linear tiny workload")
    w = workload(1)
    x, W, b = make_x(w), make_w(w), make_bias(w)
    wq, sw = qd.prepare_weights(to_dev(W))
    wqo, swo = O.prepare_weights(W)
    assert np.array_equal(host(wq), wqo) and np.array_equal(host(sw), swo)
    y = qd.int8_linear(to_dev_bf16(x), wq, sw, to_dev_bf16(b))
    yo = O.linear(x, wqo, swo, b)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "int8_linear")
    say(f"  {n} of {yo.size} outputs differ from the oracle")
    # unrotated variant
    wq0, sw0 = qd.prepare_weights(to_dev(W), block=0)
    y0 = qd.int8_linear(to_dev_bf16(x), wq0, sw0, to_dev_bf16(b), rotate_block=0)
    yo0 = O.linear(x, *O.prepare_weights(W, 0), b, block=0)
    assert_bf16_within_1ulp(bf16_bits(y0), yo0, "int8_linear unrotated")


@pytest.mark.parametrize("M", [1, 2, 255, 257, 511])
def test_int8_linear_ragged_rows(qd, O, tiles, M):
    say(f"int8_linear ragged M={M} tiles={tiles}")
    from synth import make_bias, make_w, workload
    w = workload(1)
    W, b = make_w(w), make_bias(w)
    x = _x((M, w.K), seed=700 + M, outliers=4)
    wqo, swo = O.prepare_weights(W)
    y = qd.int8_linear(to_dev_bf16(x), to_dev(wqo), to_dev(swo), to_dev_bf16(b))
    assert_bf16_within_1ulp(bf16_bits(y), O.linear(x, wqo, swo, b), "ragged")


def test_dequantize(qd, O):
    import torch
    say("dequantize")
    g = np.random.Generator(np.random.PCG64(800))
    q = g.integers(-127, 128, (37, 272), dtype=np.int64).astype(np.int8)
    s = (g.uniform(0.5, 2, 37) * 2.0 ** g.integers(-30, 5, 37)).astype(np.float32)
    d = qd.dequantize_int8(to_dev(q), to_dev(s))
    assert np.array_equal(host(d).view(np.uint32), O.dequantize(q, s, True, "f32").view(np.uint32))
    db = qd.dequantize_int8(to_dev(q), to_dev(s), torch.bfloat16)
    assert np.array_equal(bf16_bits(db), O.dequantize(q, s, True, "bf16"))
    dt = qd.dequantize_int8(to_dev(q), to_dev(s[:1]))
    assert np.array_equal(host(dt), O.dequantize(q, s[:1], False, "f32"))


def test_empty_inputs(qd):
    import torch
    say("empty inputs")
    x = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    q, s = qd.quantize_and_rotate_rowwise(x)
    assert q.shape == (0, 512) and s.shape == (0,)
    wq = torch.zeros((8, 512), dtype=torch.int8, device="cuda")
    sw = torch.ones(8, dtype=torch.float32, device="cuda")
    y = qd.int8_linear(x, wq, sw)
    assert y.shape == (0, 8)
