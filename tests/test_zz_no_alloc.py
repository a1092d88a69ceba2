"""The allocation-free entry point qd_quantize_int8_tensorwise_noalloc
(partial maxima in the library's fixed per-GPU array) against the existing
qd_quantize_int8_tensorwise (caller workspace), through the C ABI: codes and
scale bit for bit, on consecutive calls whose second input is smaller (and
has a smaller maximum, so a partial left over from the first call would
show in the scale), for each input type; and against the oracle."""
import numpy as np
import pytest

from gpu_util import host, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import quantized_diffusion_amd as q
    q.lib()
    return q


def _input(dtype, M, K, seed, amp):
    from synth import f32_to_bf16_bits
    g = np.random.Generator(np.random.PCG64(seed))
    xf = (g.standard_normal((M, K), dtype=np.float32) * np.float32(amp)).astype(np.float32)
    xf[M // 2, K // 3] = np.float32(5.0 * amp)           # the maximum in an inner row
    if dtype == "bf16":
        x = f32_to_bf16_bits(xf)
        return x, to_dev_bf16(x)
    x = xf.astype(np.float16) if dtype == "f16" else xf
    return x, to_dev(x)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_noalloc_matches_workspace_entry(qd, O, dtype):
    import torch
    # first call: more rows than the 2048 partials (every slot written);
    # second: fewer rows, a maximum 100x smaller
    for M, K, seed, amp in ((3000, 1024, 11, 100.0), (70, 528, 12, 1.0)):
        say(f"noalloc tensorwise {dtype} M={M} K={K}")
        x, xd = _input(dtype, M, K, seed, amp)
        q0, s0 = qd.quantize_int8_tensorwise(xd)
        q1 = torch.full((M, (K + 15) // 16 * 16), 99, dtype=torch.int8, device="cuda")[:, :K]
        s1 = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        qd.quantize_int8_tensorwise_noalloc(xd, q1, s1)
        torch.cuda.synchronize()
        assert host(s1).view(np.uint32)[0] == host(s0).view(np.uint32)[0], (M, host(s1)[0], host(s0)[0])
        assert torch.equal(q1, q0)
        qo, so = O.quantize_tensorwise(x, dtype)
        assert host(s1).view(np.uint32)[0] == so.view(np.uint32)[0]
        assert np.array_equal(host(q1), qo)


def test_noalloc_repeated_small_after_large(qd):
    """Calls in one stream order, large then small then large again, interleaved
    with the workspace entry point: every result equals that entry point's."""
    import torch
    shapes = [(2500, 256, 21, 50.0), (1, 16, 22, 1.0), (2049, 64, 23, 0.01), (5, 4096, 24, 3.0)]
    outs = []
    for M, K, seed, amp in shapes:
        _, xd = _input("bf16", M, K, seed, amp)
        q1 = torch.empty((M, K), dtype=torch.int8, device="cuda")
        s1 = torch.empty((1,), dtype=torch.float32, device="cuda")
        qd.quantize_int8_tensorwise_noalloc(xd, q1, s1)
        outs.append((xd, q1, s1))
    for xd, q1, s1 in outs:
        q0, s0 = qd.quantize_int8_tensorwise(xd)
        assert torch.equal(s1, s0) and torch.equal(q1, q0)
