"""Pins of the oracle against what the mathematics fixes.

Each check takes an ``Oracle`` instance and raises AssertionError on a
mismatch.  They are run against the real oracle (test_oracle_pins.py) and
against deliberately mutated copies of it (test_oracle_mutations.py), which
shows that a plausible slip -- a flipped sign, a reversed stage order, a
wrong scale formula, a dropped term, a transposed operand -- is caught.

Nothing here re-uses the oracle's code: exact rationals (fractions) and
Python integers, closed forms of the Sylvester-Hadamard matrix, the
recursive block definition H_2n = [[H_n, H_n], [H_n, -H_n]], invariants,
rounding-error bounds, and torch's own BF16 cast serve as the independent
references.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

from exact import as_frac, bf16_bits_to_float, rn32, rne_int, sylvester

U = Fraction(1, 2 ** 24)          # unit roundoff of binary32


def gamma(n: int) -> Fraction:
    return n * U / (1 - n * U)


def _unit(j):
    e = np.zeros(256, np.float32)
    e[j] = 1.0
    return e


# ---------------------------------------------------------------- rotation

def check_hadamard_closed_form(O):
    H = sylvester(256)
    for j in range(256):
        col = O.hadamard256(_unit(j)).astype(np.float64) * 16.0
        assert np.array_equal(col, H[:, j].astype(np.float64)), f"column {j}"


def check_rotation_orthogonal(O):
    R = np.stack([O.hadamard256(_unit(j)).astype(np.float64) for j in range(256)])
    assert np.array_equal(R @ R.T, np.eye(256)), "R R^T != I"
    assert np.array_equal(R, R.T), "R not symmetric"


def check_rotation_all_ones(O):
    v = O.hadamard256(np.ones(256, np.float32))
    want = np.zeros(256, np.float32)
    want[0] = 16.0
    assert np.array_equal(v, want)


def _fwht_recursive(u):
    """Sylvester recursion H_2n = [[H_n, H_n], [H_n, -H_n]] in binary32."""
    n = len(u)
    if n == 1:
        return [u[0]]
    h = n // 2
    a = _fwht_recursive(u[:h])
    b = _fwht_recursive(u[h:])
    return [a[i] + b[i] for i in range(h)] + [a[i] - b[i] for i in range(h)]


def check_rotation_recursive_definition(O):
    g = np.random.Generator(np.random.PCG64(11))
    for t in range(6):
        u = (g.standard_normal(256) * np.exp(g.uniform(-8, 8, 256))).astype(np.float32)
        want = np.array([x * np.float32(0.0625) for x in _fwht_recursive([np.float32(v) for v in u])],
                        np.float32)
        got = O.hadamard256(u)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"block {t}"


def check_rotation_error_bound(O):
    H = sylvester(256)
    g = np.random.Generator(np.random.PCG64(12))
    for t in range(3):
        u = (g.standard_normal(256) * np.exp(g.uniform(-4, 4, 256))).astype(np.float32)
        got = O.hadamard256(u)
        uf = [as_frac(v) for v in u]
        sabs = sum(abs(v) for v in uf)
        for i in range(0, 256, 7):
            exact = sum(int(H[i, k]) * uf[k] for k in range(256)) / 16
            assert abs(as_frac(got[i]) - exact) <= gamma(8) * sabs / 16, (t, i)


def check_rotation_invariants(O):
    g = np.random.Generator(np.random.PCG64(13))
    u = g.standard_normal(256).astype(np.float32)
    a = O.hadamard256(u)
    assert np.array_equal(O.hadamard256(-u).view(np.uint32), (-a).view(np.uint32))
    assert np.array_equal(O.hadamard256(u * np.float32(8.0)), a * np.float32(8.0))


def check_rotate_rows_blockwise(O):
    """Rows rotate block by block: a block-diagonal R, blocks independent."""
    g = np.random.Generator(np.random.PCG64(14))
    x = g.standard_normal((3, 1024)).astype(np.float32)
    v = O.rotate_rows(x, "f32", 256)
    H = sylvester(256).astype(np.float64) / 16.0
    for m in range(3):
        for b in range(4):
            blk = x[m, 256 * b:256 * b + 256].astype(np.float64)
            ref = H @ blk
            bound = float(gamma(8)) * np.abs(blk).sum() / 16.0 + 1e-30
            assert np.max(np.abs(v[m, 256 * b:256 * b + 256] - ref)) <= bound, (m, b)
    y = x.copy()
    y[:, 512:768] *= 3.0
    w = O.rotate_rows(y, "f32", 256)
    assert np.array_equal(w[:, :512], v[:, :512]) and np.array_equal(w[:, 768:], v[:, 768:])


def check_widening(O):
    g = np.random.Generator(np.random.PCG64(15))
    bits = g.integers(0, 1 << 16, size=(2, 512), dtype=np.uint32).astype(np.uint16)
    bits[(bits & 0x7F80) == 0x7F80] = 0x3F80          # keep finite values
    v = O.rotate_rows(bits, "bf16", 0)
    want = np.array([[bf16_bits_to_float(b) for b in row] for row in bits], np.float32)
    assert np.array_equal(v.view(np.uint32), want.view(np.uint32))
    h = g.standard_normal((2, 512)).astype(np.float16)
    h[0, :5] = np.array([6.0e-8, -6.0e-8, 65504.0, 1.0e-5, 0.0], np.float16)
    assert np.array_equal(O.rotate_rows(h, "f16", 0), h.astype(np.float32))


# ------------------------------------------------------------ quantization

def _quant_ref(row, qmax):
    amax = max(abs(as_frac(v)) for v in row)
    s = rn32(amax / qmax)
    if s == 0:
        return [0] * len(row), s
    codes = []
    for v in row:
        c = rne_int(rn32(as_frac(v) / s))
        codes.append(max(-qmax, min(qmax, c)))
    return codes, s


def check_quantize_ties(O):
    row = np.array([[127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, -1.5, 126.5, -127]], np.float32)
    q, s = O.quantize_rows(row, 127)
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 2, 4, -2, 0, 2, 0, -2, 126, -127]


def check_quantize_bruteforce(O):
    g = np.random.Generator(np.random.PCG64(16))
    rows = [g.standard_normal(24).astype(np.float32) * np.float32(10.0 ** e) for e in range(-6, 7)]
    rows += [g.uniform(-1, 1, 24).astype(np.float32) * np.float32(2.0 ** -140)]   # subnormal row
    rows += [np.zeros(24, np.float32)]
    for t in range(40):                                                             # near-tie values
        amax = np.float32(g.uniform(0.5, 300))
        s = float(rn32(as_frac(amax) / 127))
        n = g.integers(-126, 126, size=23)
        near = [np.float32((k + 0.5) * s) for k in n]
        near = [np.nextafter(v, np.float32(g.choice([-1, 1]) * np.inf)) if g.random() < 0.5 else v
                for v in near]
        rows.append(np.array([amax] + near, np.float32))
    for qmax in (127, 7):
        x = np.stack(rows)
        q, s = O.quantize_rows(x, qmax)
        for i, row in enumerate(rows):
            codes, sref = _quant_ref(row, qmax)
            assert as_frac(s[i]) == sref, (qmax, i, s[i], float(sref))
            assert q[i].tolist() == codes, (qmax, i)


def check_quantize_zero_row(O):
    q, s = O.quantize_rowwise(np.zeros((2, 512), np.uint16), "bf16", 256)
    assert np.all(q == 0) and np.all(s == 0)


def check_quantize_spike(O):
    H = sylvester(256)
    for j, c_bits in ((3, 0x4120), (300, 0xC2C8), (511, 0x3DCD)):     # 10, -100, 0.1 in BF16
        x = np.zeros((1, 512), np.uint16)
        x[0, j] = c_bits
        c = bf16_bits_to_float(c_bits)
        q, s = O.quantize_rowwise(x, "bf16", 256)
        b, jj = divmod(j, 256)
        sref = rn32(rn32(abs(as_frac(c)) / 16) / 127)
        assert as_frac(s[0]) == sref
        sign = 1 if c > 0 else -1
        assert q[0, 256 * b:256 * b + 256].tolist() == (127 * sign * H[:, jj]).tolist()
        other = 1 - b
        assert np.all(q[0, 256 * other:256 * other + 256] == 0)


def check_quantize_scale_and_sign(O):
    from synth import random_bf16
    x = random_bf16((4, 768), seed=17)
    q, s = O.quantize_rowwise(x, "bf16", 256)
    xs = x.copy()
    nz = (xs & 0x7F80) != 0                                   # normal values: add 3 to the exponent
    xs[nz] = xs[nz] + np.uint16(3 << 7)
    qs, ss = O.quantize_rowwise(xs, "bf16", 256)
    assert np.array_equal(qs, q) and np.array_equal(ss, s * np.float32(8.0))
    xn = x ^ np.uint16(0x8000)
    qn, sn = O.quantize_rowwise(xn, "bf16", 256)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)


def check_roundtrip_bound(O):
    from synth import random_bf16
    x = random_bf16((6, 1024), seed=18, scale=3.0)
    v = O.rotate_rows(x, "bf16", 256)
    q, s = O.quantize_rowwise(x, "bf16", 256)
    q2, s2 = O.quantize_rows(v, 127)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    d = O.dequantize(q, s, True, "f32")
    bound = s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -16)
    assert np.all(np.abs(v.astype(np.float64) - d.astype(np.float64)) <= bound)


def check_tensorwise_bruteforce(O):
    """Tensor-wise codes and scale against exact rationals: one amax over the
    whole tensor, s = fl(amax / 127), codes rne(fl(x / s)) clamped."""
    g = np.random.Generator(np.random.PCG64(26))
    cases = []
    for e in (-3, 0, 2):
        cases.append(g.standard_normal((5, 16)).astype(np.float32) * np.float32(10.0 ** e))
    x = np.zeros((3, 16), np.float32)                       # near-ties of the global scale
    amax = np.float32(37.5)
    s = float(rn32(as_frac(amax) / 127))
    x[0, 0] = amax
    n = g.integers(-126, 126, size=x.size - 1)
    near = [np.float32((k + 0.5) * s) for k in n]
    near = [np.nextafter(v, np.float32(g.choice([-1, 1]) * np.inf)) if g.random() < 0.5 else v for v in near]
    x.reshape(-1)[1:] = near
    cases.append(x)
    cases.append(g.uniform(-1, 1, (2, 16)).astype(np.float32) * np.float32(2.0 ** -140))   # subnormal
    cases.append(np.zeros((2, 16), np.float32))
    for x in cases:
        q, s = O.quantize_tensorwise(x, "f32")
        codes, sref = _quant_ref(x.reshape(-1), 127)
        assert as_frac(s[0]) == sref
        assert q.reshape(-1).tolist() == codes
    # BF16 input: the same definition on the widened values
    from synth import random_bf16
    xb = random_bf16((4, 32), seed=27, scale=2.0)
    q, s = O.quantize_tensorwise(xb, "bf16")
    codes, sref = _quant_ref([np.float32(bf16_bits_to_float(b)) for b in xb.reshape(-1)], 127)
    assert as_frac(s[0]) == sref and q.reshape(-1).tolist() == codes


def check_tensorwise_is_flattened_rowwise(O):
    """A tensor-wise scale is the row scale of the tensor flattened to one row;
    rows with different maxima must not get their own scales."""
    from synth import random_bf16
    x = random_bf16((6, 64), seed=28)
    x[2] = random_bf16((1, 64), seed=29, scale=40.0)[0]     # one row with a much larger amax
    q, s = O.quantize_tensorwise(x, "bf16")
    qf, sf = O.quantize_rowwise(x.reshape(1, -1), "bf16", 0)
    assert np.array_equal(q.reshape(1, -1), qf) and np.array_equal(s, sf)
    qr, sr = O.quantize_rowwise(x, "bf16", 0)
    assert not np.array_equal(q, qr)                         # per-row scales differ here
    i = np.unravel_index(np.argmax(np.abs((x.astype(np.uint32) << 16).view(np.float32))), x.shape)
    assert abs(int(q[i])) == 127


# ------------------------------------------------------------------ GEMM

def check_gemm_bruteforce(O):
    g = np.random.Generator(np.random.PCG64(19))
    for (M, K, N) in ((5, 48, 7), (3, 256, 2), (1, 16, 9)):
        a = g.integers(-128, 128, size=(M, K), dtype=np.int64).astype(np.int8)
        w = g.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
        acc = O.gemm_i32(a, w)
        assert acc.shape == (M, N)
        for m in range(M):
            for n in range(N):
                assert int(acc[m, n]) == sum(int(a[m, k]) * int(w[n, k]) for k in range(K)), (M, K, N, m, n)


def check_gemm_extremes(O):
    K = 5376
    a = np.full((2, K), 127, np.int8)
    w = np.stack([np.full(K, 127, np.int8), np.full(K, -127, np.int8)])
    acc = O.gemm_i32(a, w)
    assert acc[:, 0].tolist() == [16129 * K] * 2 and acc[:, 1].tolist() == [-16129 * K] * 2
    big = np.full((1, 140000), 127, np.int8)
    try:
        O.gemm_i32(big, big)
    except OverflowError:
        pass
    else:
        raise AssertionError("int32 overflow not reported")


# -------------------------------------------------------------- epilogue

def check_bf16_rne(O):
    import torch
    g = np.random.Generator(np.random.PCG64(20))
    f = (g.standard_normal(4096) * np.exp(g.uniform(-80, 80, 4096))).astype(np.float32)
    special = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x7F7FFFFF, 0xFF7FFFFF,
                        0x00008000, 0x00018000, 0x80000000, 0x7F800000, 0x3F80FFFF, 0x3F807FFF],
                       np.uint32).view(np.float32)
    f = np.concatenate([f, special])
    got = O.bf16_rne(f)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    nan = O.bf16_rne(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def check_epilogue_exact_order(O):
    g = np.random.Generator(np.random.PCG64(21))
    M, N = 6, 9
    acc = g.integers(-86_000_000, 86_000_000, size=(M, N)).astype(np.int32)
    sx = (g.uniform(0.5, 2, M) * 2.0 ** -7).astype(np.float32)
    sw = (g.uniform(0.5, 2, N) * 2.0 ** -12).astype(np.float32)
    from synth import random_bf16
    bias = random_bf16(N, seed=22, scale=0.1)
    t = O.epilogue_f32(acc, sx, sw, bias)
    y = O.epilogue(acc, sx, sw, bias)
    for m in range(M):
        for n in range(N):
            r = rn32(Fraction(int(acc[m, n])))
            r = rn32(r * as_frac(sx[m]))
            r = rn32(r * as_frac(sw[n]))
            b = Fraction(bf16_bits_to_float(bias[n]))
            r = rn32(r + b)
            assert as_frac(t[m, n]) == r, (m, n)
            exact = int(acc[m, n]) * as_frac(sx[m]) * as_frac(sw[n])
            assert abs(as_frac(t[m, n]) - (exact + b)) <= gamma(3) * abs(exact) * (1 + U) + U * abs(r)
    assert np.array_equal(y, O.bf16_rne(t))


def check_epilogue_closed_forms(O):
    import torch
    from synth import random_bf16
    N = 16
    bias = random_bf16(N, seed=23, scale=0.1)
    y = O.epilogue(np.zeros((2, N), np.int32), np.ones(2, np.float32), np.ones(N, np.float32), bias)
    assert np.array_equal(y, np.stack([bias, bias]))
    acc = np.array([[0, 1, -1, 255, 257, 16777217, 86_000_001, -2 ** 31 + 1]], np.int32)
    y = O.epilogue(acc, np.ones(1, np.float32), np.ones(8, np.float32), None)
    want = torch.from_numpy(acc.astype(np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, want)


# ---------------------------------------------------------- dequantization

def check_dequantize(O):
    import torch
    g = np.random.Generator(np.random.PCG64(24))
    q = g.integers(-127, 128, size=(4, 40)).astype(np.int8)
    s = (g.uniform(0.5, 2, 4) * 2.0 ** g.integers(-20, 5, 4)).astype(np.float32)
    d = O.dequantize(q, s, True, "f32")
    for m in range(4):
        for k in range(40):
            assert as_frac(d[m, k]) == rn32(int(q[m, k]) * as_frac(s[m]))
    d0 = O.dequantize(q, s[:1], False, "f32")
    assert np.array_equal(d0, O.dequantize(q, np.full(4, s[0], np.float32), True, "f32"))
    b = O.dequantize(q, s, True, "bf16")
    want = torch.from_numpy(d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, want)


# ------------------------------------------------------------ INT4 storage

def check_int4_pack(O):
    vals = np.arange(-8, 8, dtype=np.int8)
    pairs = np.array([(a, b) for a in vals for b in vals], np.int8).reshape(1, -1)
    packed = O.pack_int4(pairs)
    for i in range(pairs.shape[1] // 2):
        lo, hi = int(pairs[0, 2 * i]), int(pairs[0, 2 * i + 1])
        assert int(packed[0, i]) == ((lo & 15) | ((hi & 15) << 4))
    assert np.array_equal(O.unpack_int4(packed, pairs.shape[1]), pairs)
    assert O.pack_int4(np.array([[1, -1]], np.int8))[0, 0] == 0xF1


# ----------------------------------------------------------- whole layer

def check_linear_composition(O):
    from synth import make_bias, make_w, make_x, workload
    w = workload(1)
    x = make_x(w)[:64]
    wq, sw = O.prepare_weights(make_w(w))
    b = make_bias(w)
    y = O.linear(x, wq, sw, b)
    q, sx = O.quantize_rowwise(x)
    assert np.array_equal(y, O.epilogue(O.gemm_i32(q, wq), sx, sw, b))
    rows = np.array([0, 5, 63, 17])
    cols = np.array([0, 511, 100, 7])
    yp, accp = O.linear_points(q, sx, rows, wq, sw, b, cols)
    assert np.array_equal(yp, y[rows, cols])


def check_linear_accuracy(O):
    """End-to-end sanity (not parity): the rotated layer tracks x W^T + b in FP64,
    and rotating before quantizing beats quantizing directly on outlier data."""
    from synth import bf16_bits_to_f32, make_bias, make_w, make_x, workload
    w = workload(1)
    x = make_x(w)
    W = make_w(w)
    b = make_bias(w)
    ref = bf16_bits_to_f32(x).astype(np.float64) @ W.astype(np.float64).T + bf16_bits_to_f32(b)
    errs = {}
    for block in (256, 0):
        wq, sw = O.prepare_weights(W, block)
        y = bf16_bits_to_f32(O.linear(x, wq, sw, b, block=block)).astype(np.float64)
        errs[block] = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert errs[256] < 0.03, errs
    assert errs[256] < 0.8 * errs[0], errs


# ------------------------------------------------------- input activations

def _act_expected_bits(act: int, xs_float, dtype: str) -> np.ndarray:
    """Expected 16-bit results: the activation in 70-digit decimal arithmetic,
    rounded to nearest on the BF16/FP16 grid by exact rationals (the exact
    value is never halfway).  Large inputs are split over worker processes;
    results are cached per (act, dtype, inputs) since they do not depend on
    the oracle under test."""
    xs_float = np.asarray(xs_float, np.float32)
    key = (act, dtype, xs_float.tobytes())
    if key in _EXPECTED:
        return _EXPECTED[key]
    if len(xs_float) > 4096:
        import multiprocessing as mp
        parts = np.array_split(xs_float, 32)
        with mp.get_context("fork").Pool(min(8, os.cpu_count() or 1)) as pool:
            res = pool.starmap(_act_expected_chunk, [(act, p, dtype) for p in parts])
        out = np.concatenate(res)
    else:
        out = _act_expected_chunk(act, xs_float, dtype)
    _EXPECTED[key] = out
    return out


_EXPECTED: dict = {}


def _act_expected_chunk(act: int, xs_float, dtype: str) -> np.ndarray:
    from exact import dec_act, round_grid
    mant, emin = (7, -126) if dtype == "bf16" else (10, -14)
    out = np.empty(len(xs_float), np.uint16)
    for i, x in enumerate(xs_float):
        v = dec_act(act, float(x))
        r = Fraction(0) if v is None else round_grid(Fraction(v), mant, emin)
        if r == 0:
            neg = act != 4 and (x < 0 or (x == 0 and np.signbit(x)))
            f = -0.0 if neg else 0.0
        else:
            f = float(r)
        if dtype == "bf16":
            out[i] = np.array([f], np.float32).view(np.uint32)[0] >> 16
        else:
            out[i] = np.array([f], np.float16).view(np.uint16)[0]
    return out


def _finite_patterns(dtype: str, stride: int = 1, offset: int = 0) -> np.ndarray:
    b = np.arange(offset, 65536, stride, dtype=np.uint32).astype(np.uint16)
    expo = (b >> 7) & 0xFF if dtype == "bf16" else (b >> 10) & 0x1F
    return b[expo != (0xFF if dtype == "bf16" else 0x1F)]


def _as_float(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def _check_act(O, act, dtype, bits):
    got = O.input_act(bits, dtype, act)
    want = _act_expected_bits(act, _as_float(bits, dtype), dtype)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (act, dtype, bad.size, hex(int(bits[bad[0]])), hex(int(got[bad[0]])), hex(int(want[bad[0]])))


def check_act_relu_exact(O):
    for dtype in ("bf16", "f16"):
        b = _finite_patterns(dtype)
        got = O.input_act(b, dtype, 4)
        x = _as_float(b, dtype)
        want = np.where(x > 0, b, np.uint16(0))
        assert np.array_equal(got, want), dtype


def check_act_composition(O):
    """The layer with an activation equals the layer on the activation's
    16-bit output without one (the unfused path)."""
    from synth import random_bf16
    x = random_bf16((5, 512), seed=33, scale=2.0)
    g = np.random.Generator(np.random.PCG64(34))
    wq = g.integers(-127, 128, (24, 512), dtype=np.int64).astype(np.int8)
    sw = (g.uniform(0.5, 2, 24) * 2.0 ** -9).astype(np.float32)
    for act in (1, 2, 3, 4):
        y = O.linear(x, wq, sw, None, "bf16", 256, act=act)
        y2 = O.linear(O.input_act(x, "bf16", act), wq, sw, None, "bf16", 256)
        assert np.array_equal(y, y2), act
        q, s = O.quantize_rowwise(x, "bf16", 0, act=act)
        q2, s2 = O.quantize_rowwise(O.input_act(x, "bf16", act), "bf16", 0)
        assert np.array_equal(q, q2) and np.array_equal(s, s2), act


def slowcheck_act_all_inputs(O):
    """Every finite BF16 and FP16 input of GELU (tanh and erf forms) and SiLU."""
    for dtype in ("bf16", "f16"):
        for act in (1, 2, 3):
            _check_act(O, act, dtype, _finite_patterns(dtype))


# ------------------------------------------------------------ INT8 attention

def _lossless_rows(g, shape, exp2):
    """float32 rows that per-token quantization reproduces exactly: integers in
    [-127, 127] with a +-127 in every row, times 2^exp2 (s = 2^exp2 exactly)."""
    c = g.integers(-127, 128, shape).astype(np.float64)
    c[..., 0] = np.where(g.integers(0, 2, shape[:-1]) == 1, 127.0, -127.0)
    return (c * 2.0 ** exp2).astype(np.float32)


def check_attention_single_key(O):
    """One key: the softmax is 1, the output is that key's dequantized value row."""
    g = np.random.default_rng(31)
    q = g.standard_normal((3, 5, 64)).astype(np.float32)
    k = g.standard_normal((3, 1, 64)).astype(np.float32)
    v = (g.standard_normal((3, 1, 64)) * 3).astype(np.float32)
    out = O.attention(q, k, v, "f32")
    vc, sv = O.quantize_tokens(v, "f32")
    want = sv[:, :, None].astype(np.float64) * vc.astype(np.float64)
    assert np.array_equal(out, np.broadcast_to(want, out.shape))


def check_attention_zero_queries(O):
    """All-zero queries: every score is 0, the output is the mean of the
    dequantized value rows (per head)."""
    g = np.random.default_rng(32)
    q = np.zeros((2, 4, 128), np.float32)
    k = g.standard_normal((2, 37, 128)).astype(np.float32)
    v = g.standard_normal((2, 37, 128)).astype(np.float32)
    out = O.attention(q, k, v, "f32")
    vc, sv = O.quantize_tokens(v, "f32")
    want = (sv[:, :, None].astype(np.float64) * vc).mean(axis=1)
    assert np.allclose(out, want[:, None, :], rtol=1e-13, atol=1e-15)


def check_attention_against_sdpa(O):
    """Inputs that quantize losslessly: the oracle equals the float64 scaled
    dot-product attention of torch on the same values (an independent
    implementation), several heads, both default and explicit scales."""
    import torch
    g = np.random.default_rng(33)
    for BH, Lq, Lk, D, scale in ((2, 9, 50, 64, None), (3, 4, 17, 128, 0.3)):
        q = _lossless_rows(g, (BH, Lq, D), -9)
        k = _lossless_rows(g, (BH, Lk, D), -8)
        v = _lossless_rows(g, (BH, Lk, D), -5)
        out = O.attention(q, k, v, "f32", scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q.astype(np.float64)), torch.from_numpy(k.astype(np.float64)),
            torch.from_numpy(v.astype(np.float64)), scale=scale).numpy()
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-14), (BH, Lq, Lk, D, np.abs(out - ref).max())


def check_attention_key_permutation(O):
    """Permuting the keys together with their values leaves the output unchanged."""
    g = np.random.default_rng(34)
    q = g.standard_normal((1, 6, 64)).astype(np.float32) * 4
    k = g.standard_normal((1, 40, 64)).astype(np.float32)
    v = g.standard_normal((1, 40, 64)).astype(np.float32)
    p = g.permutation(40)
    a = O.attention(q, k, v, "f32")
    b = O.attention(q, k[:, p], v[:, p], "f32")
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def check_attention_probs(O):
    """The softmax probabilities: against torch's float64 softmax of the
    scores of losslessly quantized inputs (an independent implementation);
    rows sum to 1; and probabilities times dequantized values give the
    oracle's attention output."""
    import torch
    g = np.random.default_rng(35)
    BH, Lq, Lk, D, scale = 2, 7, 45, 64, 0.2
    q = _lossless_rows(g, (BH, Lq, D), -9)
    k = _lossless_rows(g, (BH, Lk, D), -8)
    v = g.standard_normal((BH, Lk, D)).astype(np.float32)
    qc, sq = O.quantize_tokens(q, "f32")
    kc, sk = O.quantize_tokens(k, "f32")
    vc, sv = O.quantize_tokens(v, "f32")
    P = O.attention_probs(qc, sq, kc, sk, scale)
    s = torch.from_numpy(q.astype(np.float64)) @ torch.from_numpy(k.astype(np.float64)).transpose(1, 2) * scale
    ref = torch.softmax(s, dim=-1).numpy()
    assert np.allclose(P, ref, rtol=1e-12, atol=1e-16), np.abs(P - ref).max()
    assert np.allclose(P.sum(-1), 1.0, rtol=0, atol=1e-13)
    out = O.attention_codes(qc, sq, kc, sk, vc, sv, scale)
    assert np.allclose(np.matmul(P, sv[:, :, None].astype(np.float64) * vc), out, rtol=1e-12, atol=1e-15)


CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
# Slow exhaustive checks run after the quick ones.
CHECKS += [v for k, v in sorted(globals().items()) if k.startswith("slowcheck_")]
