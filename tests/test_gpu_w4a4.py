"""GPU parity of the rotated INT4 (W4A4) path against the oracle: packing
bit-exact, INT32 accumulators of the packed-INT4 GEMM exact, BF16 outputs
within one ulp (expected bit-identical), small ragged shapes and the full
M8192/K28672/N7168 workload (sampled outputs)."""
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


def _codes(shape, seed, lo=-8, hi=8):
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(lo, hi, shape, dtype=np.int64).astype(np.int8)


@pytest.mark.parametrize("R,K", [(1, 32), (7, 96), (300, 28672)])
def test_pack_int4(qd, O, R, K):
    say(f"pack_int4 R={R} K={K}")
    q = _codes((R, K), seed=R + K)
    p = qd.pack_int4(to_dev(q))
    assert np.array_equal(host(p), O.pack_int4(q))


@pytest.mark.parametrize("M,N,K", [(1, 1, 64), (256, 256, 64), (257, 300, 512), (300, 1000, 28672), (64, 8, 1024),
                                   (300, 520, 256), (300, 520, 320), (300, 520, 384), (300, 520, 448)])
def test_int4_gemm_i32_exact(qd, O, M, N, K):
    say(f"int4 gemm i32 M={M} N={N} K={K}")
    a = _codes((M, K), seed=M * 3 + K, lo=-7)
    w = _codes((N, K), seed=N * 5 + K)
    wp = O.pack_int4(w)
    acc = qd.int4_gemm_i32(to_dev(a), to_dev(wp))
    assert np.array_equal(host(acc), O.gemm_i32(a, w))


def test_int4_gemm_largest_stride(qd, O):
    """Activation codes and packed INT4 weights whose rows lie QD_MAX_LD_GEMM
    bytes apart (the largest stride accepted): INT32 bit for bit."""
    import os
    import re
    import torch
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qdiff.h")
    ld = int(re.search(r"#define QD_MAX_LD_GEMM (\d+)", open(hdr).read()).group(1))
    M, N, K = 300, 280, 256
    say(f"int4 gemm i32 row stride {ld} M={M} N={N} K={K}")
    a = _codes((M, K), seed=830, lo=-7)
    w = _codes((N, K), seed=831)
    ab = torch.zeros((M, ld), dtype=torch.int8, device="cuda")
    wb = torch.zeros((N, ld), dtype=torch.uint8, device="cuda")
    ab[:, :K] = to_dev(a)
    wb[:, :K // 2] = to_dev(O.pack_int4(w))
    acc = qd.int4_gemm_i32(ab[:, :K], wb[:, :K // 2])
    assert np.array_equal(host(acc), O.gemm_i32(a, w))
    del ab, wb


def test_int4_scaled_mm(qd, O):
    say("int4 scaled_mm")
    from synth import random_bf16
    M, N, K = 300, 520, 1024
    g = np.random.Generator(np.random.PCG64(77))
    a = _codes((M, K), seed=78, lo=-7)
    w = _codes((N, K), seed=79, lo=-7)
    sx = (g.uniform(0.5, 2, M) * 2.0 ** -3).astype(np.float32)
    sw = (g.uniform(0.5, 2, N) * 2.0 ** -6).astype(np.float32)
    b = random_bf16(N, seed=80, scale=0.1)
    y = qd.int4_scaled_mm(to_dev(a), to_dev(sx), to_dev(O.pack_int4(w)), to_dev(sw), to_dev_bf16(b))
    n = assert_bf16_within_1ulp(bf16_bits(y), O.epilogue(O.gemm_i32(a, w), sx, sw, b), "int4_scaled_mm")
    say(f"  {n} outputs differ")


@pytest.mark.parametrize("M,K,N", [(1, 256, 8), (257, 1024, 300), (512, 2048, 1024)])
def test_convrot_w4a4_linear(qd, O, M, K, N):
    say(f"convrot_w4a4_linear M={M} K={K} N={N}")
    from synth import f32_to_bf16_bits, random_bf16
    g = np.random.Generator(np.random.PCG64(M + K + N))
    x = g.standard_normal((M, K), dtype=np.float32)
    x[:, g.choice(K, max(1, K // 100), replace=False)] *= 20
    x = f32_to_bf16_bits(x)
    W = (g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    b = random_bf16(N, seed=K, scale=0.1)
    wp, sw = qd.prepare_weights_w4a4(to_dev(W))
    wq_o, sw_o = O.prepare_weights(W, 256, qmax=7)
    assert np.array_equal(host(sw).view(np.uint32), sw_o.view(np.uint32))
    assert np.array_equal(host(wp), O.pack_int4(wq_o))
    y = qd.convrot_w4a4_linear(to_dev_bf16(x), wp, sw, to_dev_bf16(b))
    yo = O.linear(x, wq_o, sw_o, b, qmax=7)
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, "w4a4")
    say(f"  {n} outputs differ")


def test_w4a4_full_size(qd, O):
    """M8192/K28672/N7168 in the launch configuration bench.py uses."""
    import torch

    from synth import iter_w, iter_x, make_bias, workload
    w = workload(5)
    M, K, N = w.M, w.K, w.N
    dev = torch.device("cuda:0")
    say(f"full-size {w.name}")
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
    wp, sw = qd.prepare_weights_w4a4(Wd)
    del Wd
    wq_o, sw_o = O.prepare_weights(W, 256, qmax=7)
    del W
    assert np.array_equal(host(sw).view(np.uint32), sw_o.view(np.uint32))
    assert np.array_equal(host(wp), O.pack_int4(wq_o))
    say("  activation codes")
    q, s = qd.quantize_and_rotate_rowwise_int4(xd)
    qo, so = O.quantize_rowwise(x_host, "bf16", 256, qmax=7)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)
    del q
    say("  convrot_w4a4_linear")
    ws = torch.empty(qd.workspace_size(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qd.convrot_w4a4_linear(xd, wp, sw, torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev), 256, ws, y)
    g = np.random.Generator(np.random.PCG64(9005))
    rows = np.concatenate([g.integers(0, M, 8000), np.zeros(N, np.int64), np.full(N, M - 1)])
    cols = np.concatenate([g.integers(0, N, 8000), np.arange(N), np.arange(N)])
    yo, acco = O.linear_points(qo, so, rows, wq_o, sw_o, b, cols)
    ri = torch.from_numpy(rows).to(dev)
    ci = torch.from_numpy(cols).to(dev)
    n = assert_bf16_within_1ulp(bf16_bits(y[ri, ci]), yo, "w4a4 full size")
    say(f"  {n} of {yo.size} sampled outputs not bit-identical")
    aq = ws[: M * K].view(M, K).view(torch.int8)
    acc = qd.int4_gemm_i32(aq, wp)
    assert np.array_equal(host(acc[ri, ci]), acco)


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


def test_int4_scaled_mm_strided_out_no_bias_tiny_scales(qd, O):
    """Output rows 776 elements apart (whole tiles in the first tile row, a
    partial one after), no bias, subnormal and signed-zero products: every
    output bit for bit as the oracle's, nothing written between the rows."""
    say("int4 scaled_mm strided output, no bias, subnormal products")
    a, w, sx, sw = _tiny_case(90)
    M, K = a.shape
    N = w.shape[0]
    buf, y = _strided_out(M, N, 264)
    qd.int4_scaled_mm(to_dev(a), to_dev(sx), to_dev(O.pack_int4(w)), to_dev(sw), None, out=y)
    _check_exact(y, buf, N, O.epilogue(O.gemm_i32(a, w), sx, sw, None), "int4 scaled_mm")
