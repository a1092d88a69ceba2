"""Full-size workloads (8193/5376/16128, 32700/5376/16128, 14850/7168/28672)
in the launch configuration bench.py times: the GPU weight preparation and
every activation code / row scale against the oracle bit for bit, and
sampled outputs (plus whole first/last rows) against the oracle's values at
those points, INT32 accumulators bit-exact, BF16 within one ulp."""
import numpy as np
import pytest

from gpu_util import assert_bf16_within_1ulp, bf16_bits, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size_workload(O, cid):
    import torch

    import quantized_diffusion_amd as qd
    from synth import iter_w, iter_x, make_bias, workload

    w = workload(cid)
    M, K, N = w.M, w.K, w.N
    dev = torch.device("cuda:0")
    say(f"full-size {w.name}: inputs")
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

    say("  weight preparation")
    wq, sw = qd.prepare_weights(Wd)
    del Wd
    wqo, swo = O.prepare_weights(W)
    del W
    assert np.array_equal(host(sw).view(np.uint32), swo.view(np.uint32))
    assert np.array_equal(host(wq), wqo)

    say("  activation codes")
    q, s = qd.quantize_and_rotate_rowwise(xd)
    qo, so = O.quantize_rowwise(x_host, "bf16", 256)
    assert np.array_equal(host(s).view(np.uint32), so.view(np.uint32))
    assert np.array_equal(host(q), qo)
    del q

    say("  int8_linear (bench launch configuration)")
    ws = torch.empty(qd.workspace_size(M, K), dtype=torch.uint8, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qd.int8_linear(xd, wq, sw, bd, 256, ws, y)
    torch.cuda.synchronize()

    g = np.random.Generator(np.random.PCG64(9000 + cid))
    npts = 20000
    rows = g.integers(0, M, npts)
    cols = g.integers(0, N, npts)
    # whole first and last rows, and the last column
    rows = np.concatenate([rows, np.zeros(N, np.int64), np.full(N, M - 1), np.arange(M)[:: max(1, M // 512)]])
    cols = np.concatenate([cols, np.arange(N), np.arange(N), np.full(len(np.arange(M)[:: max(1, M // 512)]), N - 1)])
    yo, acco = O.linear_points(qo, so, rows, wqo, swo, b, cols)
    ri = torch.from_numpy(rows).to(dev)
    ci = torch.from_numpy(cols).to(dev)
    yg = bf16_bits(y[ri, ci])
    n = assert_bf16_within_1ulp(yg, yo, f"workload {cid}")
    say(f"  {n} of {yo.size} sampled outputs not bit-identical")

    aq = ws[: M * K].view(M, K).view(torch.int8)
    for tiles in (qd.GEMM_TILES_256x256, qd.GEMM_TILES_256x384):
        say(f"  int32 accumulators at the sampled points, tile setting {tiles}")
        qd.set_gemm_tiles(tiles)
        try:
            acc = qd.int8_gemm_i32(aq, wq)
        finally:
            qd.set_gemm_tiles(qd.GEMM_TILES_AUTO)
        assert np.array_equal(host(acc[ri, ci]), acco)
        del acc
