"""Error bound for int8_attention outputs against the oracle's float64 values.

The kernel evaluates, per query i and output dimension d,
    out = bf16( sum_j bf16(p_j) * vt_jd / sum_j p_j ),   vt_jd = bf16(fl(sv_j * vc_jd)),
with p_j = 2^(x_j c_i - m c_i), x_j = fl(acc_j * sk_j), c_i = fl(sq_i * scale * log2 e)
and a reference m that may lag the running maximum (a factor common to all
p_j cancels in the ratio), FP32 accumulation of the BF16 products (exact
products) and of the denominator.

The value operand vt is a fixed function of the codes (the documented BF16
rounding of the dequantized values), so its effect is computed exactly:
with the oracle's softmax probabilities P (rows summing to 1), A = P v is
the oracle's output and At = P vt the exact output on the rounded values.
What remains is bounded term by term, every rounding being a relative
perturbation of one term or of the ratio:
  * p_j: theta from the FP32 exponent argument and the exp2 approximation,
    then 2^-8 from the BF16 rounding;
  * sums: gamma_n = n u / (1 - n u) for n terms in any order;
  * the quotient: 3 u (reciprocal and product), then 2^-8 (BF16 output).
With Wt = P |vt|:  |out - A| <= |At - A| + d + 2^-8 (|A| + |At - A| + d),
d = (e1 + |At| e2) / (1 - e2) (+ 3 u), e1 = (tau + gamma (1 + tau)) Wt,
e2 = theta + gamma, tau = (1 + theta)(1 + 2^-8) - 1.  This is a rigorous
bound for the stated arithmetic, with no factor of slack.  Test
infrastructure only.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24    # binary32 unit roundoff
BU = 2.0 ** -8    # bfloat16 unit roundoff
LOG2E = 1.4426950408889634


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest BF16 (ties to even), returned as float32."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def rounded_values(vc, sv) -> np.ndarray:
    """vt = bf16(fl32(sv * vc)) [BH, Lk, D] as float64 (exact)."""
    prod = (vc.astype(np.float32) * sv.astype(np.float32)[:, :, None]).astype(np.float32)
    return bf16_round(prod).astype(np.float64)


def score_bound(qc, sq, kc, sk, scale) -> np.ndarray:
    """Upper bound of |score| * log2(e) per query [BH, Lq] (Cauchy-Schwarz on
    the dequantized query and the largest dequantized key of its head)."""
    qn = np.sqrt((qc.astype(np.float64) ** 2).sum(-1)) * sq.astype(np.float64)
    kn = (np.sqrt((kc.astype(np.float64) ** 2).sum(-1)) * sk.astype(np.float64)).max(axis=1)
    return qn * kn[:, None] * abs(scale) * LOG2E


def attention_bound(want, P, qc, sq, kc, sk, vc, sv, scale) -> np.ndarray:
    """Per-output bound [BH, Lq, D] of |gpu - want| (see the module text).
    want: the oracle's output; P: the oracle's probabilities [BH, Lq, Lk]."""
    Lk = kc.shape[1]
    vt = rounded_values(vc, sv)
    At = np.matmul(P, vt)
    Wt = np.matmul(P, np.abs(vt))
    # float64 evaluation of At (relative 2^-53 per term, any order)
    dv = np.abs(At - want) + 2.0 ** -44 * Wt
    smax = score_bound(qc, sq, kc, sk, scale)[:, :, None]          # base-2 units
    # absolute error of the base-2 exponent's argument: the key-scale product,
    # the query factor, the reference term and the fused multiply-add, each a
    # few units of roundoff of magnitudes below smax (the reference lags the
    # maximum by at most 8)
    eta = 8.0 * U * (2.0 * smax + 16.0)
    theta = np.expm1(eta * np.log(2.0)) + 2.0 ** -21                  # + exp2 approximation
    n = Lk + 128
    gamma = n * U / (1.0 - n * U)
    tau = (1.0 + theta) * (1.0 + BU) - 1.0
    e1 = (tau + gamma * (1.0 + tau)) * Wt
    e2 = theta + gamma
    at = np.abs(At)
    d = (e1 + at * e2) / (1.0 - e2)
    d = d + 3.0 * U * (at + d)
    # underflow of tiny probabilities (absolute, far below the rest)
    d = d + Lk * 2.0 ** -126 * (np.abs(vt).max(axis=1)[:, None, :] + 1.0)
    a = np.abs(want)
    return dv + d + BU * (a + dv + d) + 2.0 ** -133


def kernel_model(qc, sq, kc, sk, vc, sv, scale) -> np.ndarray:
    """A CPU model of the kernel's arithmetic (FP32 scores and exponent,
    BF16 probabilities and values, FP32 sums), for checking that the bound
    holds for a faithful evaluation; float64 [BH, Lq, D]."""
    BH, Lq, D = qc.shape
    out = np.empty((BH, Lq, D), np.float64)
    c = np.float32(np.float32(scale) * np.float32(LOG2E))
    vt = rounded_values(vc, sv).astype(np.float32)
    for h in range(BH):
        acc = qc[h].astype(np.int64) @ kc[h].astype(np.int64).T                 # exact
        x = acc.astype(np.float32) * sk[h].astype(np.float32)[None, :]
        sqc = (sq[h].astype(np.float32) * c).astype(np.float32)[:, None]
        m = x.max(axis=1, keepdims=True)
        p = np.exp2((x * sqc - m * sqc).astype(np.float32)).astype(np.float32)
        num = bf16_round(p) @ vt[h]                                              # float32
        den = p.sum(axis=1, dtype=np.float32)[:, None]
        out[h] = bf16_round((num * (np.float32(1.0) / den)).astype(np.float32)).astype(np.float64)
    return out
