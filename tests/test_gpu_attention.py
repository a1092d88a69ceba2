"""GPU parity of int8_attention, through the C ABI, against the oracle: the
per-token codes and scales in the workspace bit for bit, and every output
within the rigorous bound derived from the kernel's rounding steps
(tests/attention_bound.py: the dequantized values' BF16 rounding evaluated
exactly with the oracle's softmax probabilities, the probabilities' BF16
rounding, the FP32 sums and the BF16 output bounded term by term, no slack).
On the CPU, tests/test_attention_bound.py shows that this bound rejects the
oracle's output with one key or one 64-key block dropped."""
import numpy as np
import pytest

from attention_bound import attention_bound
from gpu_util import host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qd():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import quantized_diffusion_amd as q
    q.lib()
    return q


def _bits_of(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(shape_q, shape_k, seed, dtype="bf16", qscale=1.0):
    import torch
    g = np.random.Generator(np.random.PCG64(seed))
    mk = lambda shp, sc: (g.standard_normal(shp) * sc).astype(np.float32)
    q, k, v = mk(shape_q, qscale), mk(shape_k, 1.0), mk(shape_k, 1.5)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    dev = [torch.from_numpy(a).to(tdt).cuda() for a in (q, k, v)]
    host_in = [(_bits_of(t) if dtype == "bf16" else t.cpu().numpy()) for t in dev]
    return dev, host_in


def _check(qd, O, dev, host_in, dtype, scale=0.0, what=""):
    import torch
    q, k, v = dev
    BH, Lq, D = q.shape
    Lk = k.shape[1]
    ws = torch.empty(qd.attention_workspace_size(BH, Lq, Lk, D), dtype=torch.uint8, device="cuda")
    out = qd.int8_attention(q, k, v, scale, workspace=ws)
    # codes and scales in the workspace (layout of qdiff.h)
    qc, sq = O.quantize_tokens(host_in[0], dtype)
    kc, sk = O.quantize_tokens(host_in[1], dtype)
    vc, sv = O.quantize_tokens(host_in[2], dtype)
    w = host(ws)
    al = lambda n: (n + 255) // 256 * 256
    off = 0
    for arr, n in ((qc, BH * Lq * D), (kc, BH * Lk * D), (vc, BH * Lk * D)):
        assert np.array_equal(w[off:off + n].view(np.int8).reshape(arr.shape), arr), f"{what}: codes"
        off += al(n)
    for arr, n in ((sq, BH * Lq), (sk, BH * Lk), (sv, BH * Lk)):
        assert np.array_equal(w[off:off + 4 * n].view(np.uint32).reshape(arr.shape), arr.view(np.uint32)), \
            f"{what}: scales"
        off += al(4 * n)
    sc = None if scale <= 0 else scale
    want = O.attention_codes(qc, sq, kc, sk, vc, sv, sc)
    P = O.attention_probs(qc, sq, kc, sk, sc)
    got = _bits_of(out).astype(np.uint32) << 16
    got = got.view(np.float32).astype(np.float64)
    bound = attention_bound(want, P, qc, sq, kc, sk, vc, sv, 1.0 / np.sqrt(D) if sc is None else sc)
    err = np.abs(got - want)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{what}: {len(bad)} outputs outside the bound, first {tuple(bad[0])}: " \
                          f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]} bound {bound[tuple(bad[0])]}"
    say(f"  {what}: max |err| / bound = {float((err / np.maximum(bound, 1e-300)).max()):.3f}, "
        f"median bound / |exact| = {float(np.median(bound / np.maximum(np.abs(want), 1e-300))):.3f}")


# Lk spans: a tail block alone, whole blocks only (1, 3 and 5 of them: the
# kernel stages two blocks ahead and synchronises after every second block),
# whole blocks plus a tail for both parities of the block count
@pytest.mark.parametrize("BH,Lq,Lk,D", [(1, 1, 1, 64), (2, 130, 200, 64), (3, 257, 64, 128), (1, 128, 1000, 128),
                                        (2, 64, 63, 128), (1, 300, 4097, 128), (4, 129, 129, 64),
                                        (1, 70, 192, 128), (2, 40, 320, 64)])
def test_attention_bf16(qd, O, BH, Lq, Lk, D):
    say(f"int8_attention bf16 BH={BH} Lq={Lq} Lk={Lk} D={D}")
    dev, h = _inputs((BH, Lq, D), (BH, Lk, D), seed=BH * 1000 + Lq + Lk + D)
    _check(qd, O, dev, h, "bf16", what=f"{BH}x{Lq}x{Lk}x{D}")


@pytest.mark.parametrize("dtype", ["f16", "f32"])
def test_attention_other_dtypes(qd, O, dtype):
    say(f"int8_attention {dtype}")
    dev, h = _inputs((2, 77, 128), (2, 150, 128), seed=41, dtype=dtype)
    _check(qd, O, dev, h, dtype, what=dtype)


def test_attention_explicit_scale_and_peaky_softmax(qd, O):
    """A large score scale: the softmax is nearly one-hot for most queries."""
    say("int8_attention explicit scale, peaky")
    dev, h = _inputs((1, 200, 128), (1, 333, 128), seed=42, qscale=4.0)
    _check(qd, O, dev, h, "bf16", scale=0.5, what="scale 0.5")


def test_attention_zero_queries(qd, O):
    """Zero queries: uniform softmax, the mean of the dequantized values."""
    import torch
    say("int8_attention zero queries")
    dev, h = _inputs((2, 40, 64), (2, 90, 64), seed=43)
    dev[0].zero_()
    h[0] = np.zeros_like(h[0])
    _check(qd, O, dev, h, "bf16", what="zero q")


def test_attention_codes_entry_matches(qd, O):
    """The codes-only entry point on the workspace's codes gives the same bits."""
    import torch
    say("int8_attention_codes == int8_attention")
    dev, h = _inputs((2, 150, 128), (2, 260, 128), seed=46)
    q, k, v = dev
    BH, Lq, D = q.shape
    Lk = k.shape[1]
    ws = torch.empty(qd.attention_workspace_size(BH, Lq, Lk, D), dtype=torch.uint8, device="cuda")
    y = qd.int8_attention(q, k, v, workspace=ws)
    al = lambda n: (n + 255) // 256 * 256
    o = [0]
    def take(n, dt, shape):
        t = ws[o[0]:o[0] + n].view(dt).view(shape)
        o[0] += al(n)
        return t
    qc = take(BH * Lq * D, torch.int8, (BH, Lq, D))
    kc = take(BH * Lk * D, torch.int8, (BH, Lk, D))
    vc = take(BH * Lk * D, torch.int8, (BH, Lk, D))
    sq = take(4 * BH * Lq, torch.float32, (BH, Lq))
    sk = take(4 * BH * Lk, torch.float32, (BH, Lk))
    sv = take(4 * BH * Lk, torch.float32, (BH, Lk))
    y2 = qd.int8_attention_codes(qc, sq, kc, sk, vc, sv)
    assert torch.equal(y, y2)


def test_attention_empty_queries(qd):
    import torch
    q = torch.empty((1, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((1, 5, 64), device="cuda").to(torch.bfloat16)
    out = qd.int8_attention(q, k, k)
    assert out.shape == (1, 0, 64)


def test_attention_large_sampled(qd, O):
    """BH=8 x L=4096 x D=128: sampled query rows against the oracle."""
    import torch
    say("int8_attention 8x4096x4096x128, sampled rows")
    dev, h = _inputs((8, 4096, 128), (8, 4096, 128), seed=44)
    q, k, v = dev
    out = qd.int8_attention(q, k, v)
    g = np.random.Generator(np.random.PCG64(45))
    rows = np.unique(np.concatenate([g.integers(0, 4096, 60), [0, 4095, 127, 128]]))
    qc, sq = O.quantize_tokens(h[0], "bf16")
    kc, sk = O.quantize_tokens(h[1], "bf16")
    vc, sv = O.quantize_tokens(h[2], "bf16")
    want = O.attention_codes(qc[:, rows], sq[:, rows], kc, sk, vc, sv)
    P = O.attention_probs(qc[:, rows], sq[:, rows], kc, sk)
    got = (_bits_of(out[:, torch.from_numpy(rows).cuda()]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = attention_bound(want, P, qc[:, rows], sq[:, rows], kc, sk, vc, sv, 1.0 / np.sqrt(128))
    err = np.abs(got - want)
    assert np.all(err <= bound), f"{int((err > bound).sum())} sampled outputs outside the bound"
    say(f"  max |err| / bound = {float((err / bound).max()):.3f}")


def test_attention_d64_long_sampled(qd, O):
    """D = 64 over long sequences (4 heads x 8192 queries x 8192 keys): rows
    of every head (first and last query, both sides of a workgroup's
    384-query boundary, random ones) against the oracle within the bound."""
    import torch
    BH, L, D = 4, 8192, 64
    say(f"int8_attention {BH}x{L}x{L}x{D}, sampled rows")
    dev, h = _inputs((BH, L, D), (BH, L, D), seed=47)
    q, k, v = dev
    out = qd.int8_attention(q, k, v)
    g = np.random.Generator(np.random.PCG64(48))
    rows = np.unique(np.concatenate([g.integers(0, L, 24), [0, 383, 384, L - 1]]))
    qc, sq = O.quantize_tokens(h[0], "bf16")
    kc, sk = O.quantize_tokens(h[1], "bf16")
    vc, sv = O.quantize_tokens(h[2], "bf16")
    want = O.attention_codes(qc[:, rows], sq[:, rows], kc, sk, vc, sv)
    P = O.attention_probs(qc[:, rows], sq[:, rows], kc, sk)
    got = (_bits_of(out[:, torch.from_numpy(rows).cuda()]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = attention_bound(want, P, qc[:, rows], sq[:, rows], kc, sk, vc, sv, 1.0 / np.sqrt(D))
    err = np.abs(got - want)
    assert np.all(err <= bound), f"{int((err > bound).sum())} sampled outputs outside the bound"
    say(f"  max |err| / bound = {float((err / bound).max()):.3f}")


def test_attention_full_size_sampled(qd, O):
    """The benchmark's workload, 40 heads x 16384 tokens x 128 (BF16 N(0, 1)
    inputs drawn as the benchmark draws them), in its launch configuration:
    rows of three heads (first, middle, last; the first and last query, both
    sides of a workgroup's 384-query boundary and random ones) against the
    oracle within the bound."""
    import torch
    BH, L, D = 40, 16384, 128
    say(f"int8_attention {BH}x{L}x{L}x{D}, sampled rows of three heads")
    gen = torch.Generator(device="cuda").manual_seed(1234)
    q, k, v = (torch.randn((BH, L, D), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
    ws = torch.empty(qd.attention_workspace_size(BH, L, L, D), dtype=torch.uint8, device="cuda")
    out = qd.int8_attention(q, k, v, workspace=ws)
    g = np.random.Generator(np.random.PCG64(46))
    rows = np.unique(np.concatenate([g.integers(0, L, 18), [0, 383, 384, L - 1]]))
    worst = 0.0
    for hd in (0, 17, BH - 1):
        hq, hk, hv = (_bits_of(t[hd:hd + 1]) for t in (q, k, v))
        qc, sq = O.quantize_tokens(hq, "bf16")
        kc, sk = O.quantize_tokens(hk, "bf16")
        vc, sv = O.quantize_tokens(hv, "bf16")
        want = O.attention_codes(qc[:, rows], sq[:, rows], kc, sk, vc, sv)
        P = O.attention_probs(qc[:, rows], sq[:, rows], kc, sk)
        sel = out[hd:hd + 1, torch.from_numpy(rows).cuda()]
        got = (_bits_of(sel).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        bound = attention_bound(want, P, qc[:, rows], sq[:, rows], kc, sk, vc, sv, 1.0 / np.sqrt(D))
        err = np.abs(got - want)
        assert np.all(err <= bound), f"head {hd}: {int((err > bound).sum())} sampled outputs outside the bound"
        worst = max(worst, float((err / bound).max()))
    say(f"  max |err| / bound = {worst:.3f}")
