"""GPU parity of W4A4 on the FP6 matrix path, through the C ABI, against the
oracle: every value of the FP6 operands the GPU writes, decoded by the tests
from the format's description, equals the oracle's INT4 code; the exact sums of the FP6
GEMM against the oracle's INT32 GEMM of the same INT4 codes bit for bit, and
BF16 outputs within one BF16 ulp (identical to the INT8-path results)."""
import numpy as np
import pytest

from fp6_format import assert_fp6_codes
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


def _codes(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(-7, 8, shape, dtype=np.int64).astype(np.int8)


@pytest.mark.parametrize("R,K", [(1, 64), (40, 192), (300, 28672)])
def test_pack_fp6(qd, O, R, K):
    say(f"pack_fp6 R={R} K={K}")
    q = _codes((R, K), 800 + R)
    p = qd.pack_fp6(to_dev(q))
    assert p.shape == (R, 3 * K // 4)
    assert_fp6_codes(host(p), q, "pack_fp6")


def test_fp6_gemm_largest_stride(qd, O):
    """Row-major FP6 operands whose rows lie QD_MAX_LD_GEMM bytes apart (the
    largest stride accepted): exact sums bit for bit."""
    import os
    import re
    import torch
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qdiff.h")
    ld = int(re.search(r"#define QD_MAX_LD_GEMM (\d+)", open(hdr).read()).group(1))
    M, N, K = 300, 280, 256
    say(f"fp6 gemm i32 row stride {ld} M={M} N={N} K={K}")
    a = _codes((M, K), 820)
    w = _codes((N, K), 821)
    ab = torch.zeros((M, ld), dtype=torch.uint8, device="cuda")
    wb = torch.zeros((N, ld), dtype=torch.uint8, device="cuda")
    ab[:, :3 * K // 4] = qd.pack_fp6(to_dev(a))
    wb[:, :3 * K // 4] = qd.pack_fp6(to_dev(w))
    acc = qd.fp6_gemm_i32(ab[:, :3 * K // 4], wb[:, :3 * K // 4], K)
    assert np.array_equal(host(acc), O.gemm_i32(a, w))
    del ab, wb


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (256, 256, 128), (257, 300, 512), (64, 8, 1024),
                                   (300, 520, 256), (300, 520, 384), (300, 520, 640), (257, 264, 768),
                                   (513, 264, 256), (300, 1000, 28672)])
def test_fp6_gemm_exact(qd, O, M, N, K):
    say(f"fp6 gemm i32 M={M} N={N} K={K}")
    a = _codes((M, K), 810 + M + K)
    w = _codes((N, K), 811 + N + K)
    acc = qd.fp6_gemm_i32(qd.pack_fp6(to_dev(a)), qd.pack_fp6(to_dev(w)), K)
    assert np.array_equal(host(acc), O.gemm_i32(a, w))


def test_fp6_gemm_extremes(qd, O):
    """|sum| up to 49 K at K = 28672 (1 404 928), both signs."""
    say("fp6 gemm extremes K=28672")
    K = 28672
    a = np.full((40, K), 7, np.int8)
    a[1::2] = -7
    w = np.full((33, K), 7, np.int8)
    w[::3] = -7
    acc = qd.fp6_gemm_i32(qd.pack_fp6(to_dev(a)), qd.pack_fp6(to_dev(w)), K)
    ref = O.gemm_i32(a, w)
    assert int(np.abs(ref).max()) == 49 * K
    assert np.array_equal(host(acc), ref)


@pytest.mark.parametrize("M,N,K", [(256, 512, 512), (257, 264, 1024), (77, 1000, 256)])
def test_fp6_scaled_mm(qd, O, M, N, K):
    say(f"fp6 scaled_mm M={M} N={N} K={K}")
    g = np.random.Generator(np.random.PCG64(820 + M))
    a = _codes((M, K), 821 + M)
    w = _codes((N, K), 822 + N)
    sx = (g.uniform(0.5, 2.0, M) * 2.0 ** -3).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, N) * 2.0 ** -8).astype(np.float32)
    from synth import random_bf16
    b = random_bf16(N, seed=823, scale=0.1)
    y = qd.fp6_scaled_mm(qd.pack_fp6(to_dev(a)), to_dev(sx), qd.pack_fp6(to_dev(w)), to_dev(sw), K,
                         to_dev_bf16(b))
    yo = O.epilogue(O.gemm_i32(a, w), sx, sw, b)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "fp6 scaled_mm")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


@pytest.mark.parametrize("M,K,N", [(1, 256, 8), (257, 1024, 300), (512, 2048, 1024)])
def test_convrot_w4a4_linear_fp6(qd, O, M, K, N):
    import torch
    say(f"convrot_w4a4_linear_fp6 M={M} K={K} N={N}")
    from synth import f32_to_bf16_bits, random_bf16
    g = np.random.Generator(np.random.PCG64(830 + M))
    x = f32_to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    b = random_bf16(N, seed=831, scale=0.1)
    w6, sw = qd.prepare_weights_w4a4_fp6(to_dev(wf))
    y = qd.convrot_w4a4_linear_fp6(to_dev_bf16(x), w6, sw, to_dev_bf16(b))
    wq_o, sw_o = O.prepare_weights(wf, 256, qmax=7)
    yo = O.linear(x, wq_o, sw_o, b, "bf16", 256, qmax=7)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "w4a4 fp6")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")
    # the INT8 path gives the same outputs
    wp, sw2 = qd.prepare_weights_w4a4(to_dev(wf))
    y8 = qd.convrot_w4a4_linear(to_dev_bf16(x), wp, sw2, to_dev_bf16(b))
    assert torch.equal(y, y8)


def test_w4a4_fp6_full_size(qd, O):
    """M8192/K28672/N7168 in the launch configuration bench.py --fp6 uses."""
    import torch

    from synth import iter_w, iter_x, make_bias, workload
    w = workload(5)
    M, K, N = w.M, w.K, w.N
    dev = torch.device("cuda:0")
    say(f"full-size fp6 {w.name}")
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
    w6, sw = qd.prepare_weights_w4a4_fp6(Wd)
    del Wd
    wq_o, sw_o = O.prepare_weights(W, 256, qmax=7)
    del W
    assert np.array_equal(host(sw).view(np.uint32), sw_o.view(np.uint32))
    assert_fp6_codes(host(w6), wq_o, "fp6 weights")
    say("  convrot_w4a4_linear_fp6")
    ws = torch.empty(qd.w4a4_fp6_workspace_size(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qd.convrot_w4a4_linear_fp6(xd, w6, sw, torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev), 256,
                               ws, y)
    qo, so = O.quantize_rowwise(x_host, "bf16", 256, qmax=7)
    g = np.random.Generator(np.random.PCG64(9006))
    rows = np.concatenate([g.integers(0, M, 8000), np.zeros(N, np.int64), np.full(N, M - 1)])
    cols = np.concatenate([g.integers(0, N, 8000), np.arange(N), np.arange(N)])
    yo, acco = O.linear_points(qo, so, rows, wq_o, sw_o, b, cols)
    ri = torch.from_numpy(rows).to(dev)
    ci = torch.from_numpy(cols).to(dev)
    n = assert_bf16_within_1ulp(bf16_bits(y[ri, ci]), yo, "w4a4 fp6 full size")
    say(f"  {n} of {yo.size} sampled outputs not bit-identical")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("M,K", [(1, 256), (33, 1280), (300, 28672), (2, 65536)])
def test_quantize_fp6_direct(qd, O, dtype, M, K):
    """The rotating INT4 quantizer writing FP6 directly: its scales equal the
    oracle's bit for bit and its FP6 values decode to the oracle's codes."""
    say(f"quantize fp6 direct {dtype} M={M} K={K}")
    g = np.random.Generator(np.random.PCG64(840 + M + K))
    xf = g.standard_normal((M, K), dtype=np.float32)
    xf[:, g.choice(K, size=max(1, K // 100), replace=False)] *= 20
    if dtype == "bf16":
        from synth import f32_to_bf16_bits
        x = f32_to_bf16_bits(xf)
        xd = to_dev_bf16(x)
    else:
        x = xf.astype(np.float16)
        xd = to_dev(x)
    q6, s = qd.quantize_and_rotate_rowwise_fp6(xd)
    qo, so = O.quantize_rowwise(x, dtype, 256, qmax=7)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert_fp6_codes(host(q6), qo, "quantize fp6")


def test_convrot_w4a4_linear_fp6_f32_input(qd, O):
    """FP32 activations take the two-step route (INT4 codes, then packing)."""
    say("convrot_w4a4_linear_fp6 f32 input")
    g = np.random.Generator(np.random.PCG64(850))
    M, K, N = 70, 512, 136
    x = g.standard_normal((M, K)).astype(np.float32)
    wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    w6, sw = qd.prepare_weights_w4a4_fp6(to_dev(wf))
    y = qd.convrot_w4a4_linear_fp6(to_dev(x), w6, sw)
    wq_o, sw_o = O.prepare_weights(wf, 256, qmax=7)
    yo = O.linear(x, wq_o, sw_o, None, "f32", 256, qmax=7)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "w4a4 fp6 f32 input")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


def _tiny_case(seed):
    """INT4 codes with row scales 2^-60, 2^-70, 2^-80 in turn and column
    scales near 2^-66: products from normal through subnormal to zero, both
    signs (zero rows and rows of small sums included), no bias."""
    M, N, K = 300, 512, 512
    g = np.random.Generator(np.random.PCG64(seed))
    a = g.integers(-7, 8, (M, K), dtype=np.int64).astype(np.int8)
    w = g.integers(-7, 8, (N, K), dtype=np.int64).astype(np.int8)
    a[::7] = 0
    a[1::5, ::2] = 1
    sx = (g.uniform(0.5, 2.0, M) * 2.0 ** (-60.0 - 10.0 * (np.arange(M) % 3))).astype(np.float32)
    sw = (g.uniform(0.5, 2.0, N) * 2.0 ** -66).astype(np.float32)
    return a, w, sx, sw


def _strided_out(M, N, pad):
    import torch
    buf = torch.full((M, N + pad), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return buf, buf[:, :N]


def _check_exact(y, buf, N, want, what):
    import torch
    got = bf16_bits(y).reshape(-1)
    want = want.reshape(-1)
    assert int((want == 0x8000).sum()) > 1000 and int((want == 0).sum()) > 1000
    assert int((((want & 0x7F80) == 0) & ((want & 0x7F) != 0)).sum()) > 1000
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} outputs differ, first at {bad[0]}: {got[bad[0]]:#06x} vs {want[bad[0]]:#06x}"
    assert bool((buf[:, N:].view(torch.int16) == -1).all()), f"{what}: writes outside the output rows"


def test_fp6_scaled_mm_strided_out_no_bias_tiny_scales(qd, O):
    """Output rows 776 elements apart (whole tiles in the first tile row, a
    partial one after), no bias, subnormal and signed-zero products: every
    output bit for bit as the oracle's, nothing written between the rows."""
    say("fp6 scaled_mm strided output, no bias, subnormal products")
    a, w, sx, sw = _tiny_case(830)
    M, K = a.shape
    N = w.shape[0]
    buf, y = _strided_out(M, N, 264)
    qd.fp6_scaled_mm(qd.pack_fp6(to_dev(a)), to_dev(sx), qd.pack_fp6(to_dev(w)), to_dev(sw), K, None, out=y)
    _check_exact(y, buf, N, O.epilogue(O.gemm_i32(a, w), sx, sw, None), "fp6 scaled_mm")
