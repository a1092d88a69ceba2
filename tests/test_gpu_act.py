"""GPU parity of the input activation folded into the quantizer
(int8_linear(input_act=...)), through the C ABI, against the oracle: every
16-bit input value of each activation bit for bit, codes and row scales of
act(x) bit for bit, BF16 layer outputs within one BF16 ulp."""
import numpy as np
import pytest

from gpu_util import assert_bf16_within_1ulp, bf16_bits, host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

ACTS = {"gelu_tanh": 1, "gelu_erf": 2, "silu": 3, "relu": 4}


@pytest.fixture(scope="module")
def qd():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import quantized_diffusion_amd as q
    q.lib()
    return q


def _finite(dtype):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    expo = (b >> 7) & 0xFF if dtype == "bf16" else (b >> 10) & 0x1F
    return b[expo != (0xFF if dtype == "bf16" else 0x1F)]


def _dev16(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def _bits16(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("act", list(ACTS))
def test_input_act_every_value(qd, O, act, dtype):
    """All finite inputs of the type, the device's activation against the oracle's."""
    say(f"input_act {act} {dtype}: every finite value")
    b = _finite(dtype)
    got = _bits16(qd.input_act(_dev16(b, dtype), ACTS[act]))
    want = O.input_act(b, dtype, ACTS[act])
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} values differ, first x={hex(int(b[bad[0]]))} got {hex(int(got[bad[0]]))} want {hex(int(want[bad[0]]))}"


def _x(shape, seed, scale=1.5):
    from synth import f32_to_bf16_bits
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    x[:, g.choice(shape[1], size=max(1, shape[1] // 100), replace=False)] *= 20
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("act", list(ACTS))
@pytest.mark.parametrize("M,K,block", [(257, 5376, 256), (3, 512, 256), (64, 528, 0), (2, 28672, 256)])
def test_quantize_rowwise_act(qd, O, act, M, K, block):
    say(f"quantize_rowwise_act {act} M={M} K={K} block={block}")
    x = _x((M, K), seed=700 + M + K + ACTS[act])
    q, s = qd.quantize_rowwise_act(to_dev_bf16(x), ACTS[act], block)
    qo, so = O.quantize_rowwise(x, "bf16", block, act=ACTS[act])
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


@pytest.mark.parametrize("act", ["gelu_tanh", "silu"])
def test_quantize_rowwise_act_f16(qd, O, act):
    say(f"quantize_rowwise_act {act} f16")
    g = np.random.Generator(np.random.PCG64(710))
    x = (g.standard_normal((33, 1280)) * 2).astype(np.float16)
    q, s = qd.quantize_rowwise_act(to_dev(x), ACTS[act], 256)
    qo, so = O.quantize_rowwise(x, "f16", 256, act=ACTS[act])
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)


@pytest.mark.parametrize("act", list(ACTS))
@pytest.mark.parametrize("M,K,N", [(256, 512, 512), (300, 1024, 264)])
def test_int8_linear_act(qd, O, act, M, K, N):
    say(f"int8_linear_act {act} M={M} K={K} N={N}")
    x = _x((M, K), seed=720 + M + ACTS[act])
    g = np.random.Generator(np.random.PCG64(721 + N))
    wf = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    wq, sw = O.prepare_weights(wf)
    from synth import random_bf16
    b = random_bf16(N, seed=722, scale=0.1)
    y = qd.int8_linear_act(to_dev_bf16(x), to_dev(wq), to_dev(sw), to_dev_bf16(b), ACTS[act], 256)
    yo = O.linear(x, wq, sw, b, "bf16", 256, act=ACTS[act])
    n = assert_bf16_within_1ulp(bf16_bits(y), yo, f"int8_linear_act {act}")
    say(f"  {n} of {yo.size} outputs differ from the oracle (allowed: 1 ulp)")


def test_int8_linear_act_none_is_int8_linear(qd, O):
    import torch
    say("int8_linear_act(NONE) == int8_linear")
    x = _x((100, 768), seed=730)
    g = np.random.Generator(np.random.PCG64(731))
    wq = g.integers(-127, 128, (200, 768), dtype=np.int64).astype(np.int8)
    sw = (g.uniform(0.5, 2, 200) * 2.0 ** -9).astype(np.float32)
    y1 = qd.int8_linear_act(to_dev_bf16(x), to_dev(wq), to_dev(sw), None, 0, 256)
    y2 = qd.int8_linear(to_dev_bf16(x), to_dev(wq), to_dev(sw), None, 256)
    assert torch.equal(y1, y2)


def test_act_full_size_codes(qd, O):
    """GELU (tanh) folded into the quantizer on the M8193/K5376 activations:
    every code and row scale."""
    from synth import make_x, workload
    w = workload(2)
    say(f"act full size {w.name}")
    x = make_x(w)
    q, s = qd.quantize_rowwise_act(to_dev_bf16(x), ACTS["gelu_tanh"], 256)
    qo, so = O.quantize_rowwise(x, "bf16", 256, act=ACTS["gelu_tanh"])
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)
