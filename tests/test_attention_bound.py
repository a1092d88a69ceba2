"""The attention parity bound (tests/attention_bound.py) on the CPU: a model
of the kernel's arithmetic stays inside it, the oracle's output with one key
or one 64-key block dropped falls outside it (so the GPU test can tell a
kernel that skips keys from a correct one), and on the long-sequence case it
is well below the outputs' own magnitude."""
import numpy as np
import pytest

import attention_bound as AB
from synth import f32_to_bf16_bits


def _case(O, BH, Lq, Lk, D, seed, qscale=1.0):
    """The GPU test's input recipe: q, k ~ N(0, 1) (q scaled), v ~ N(0, 1.5), BF16."""
    g = np.random.Generator(np.random.PCG64(seed))
    mk = lambda shp, sc: f32_to_bf16_bits((g.standard_normal(shp) * sc).astype(np.float32))
    q, k, v = mk((BH, Lq, D), qscale), mk((BH, Lk, D), 1.0), mk((BH, Lk, D), 1.5)
    qc, sq = O.quantize_tokens(q)
    kc, sk = O.quantize_tokens(k)
    vc, sv = O.quantize_tokens(v)
    return qc, sq, kc, sk, vc, sv


def _bound(O, c, scale):
    qc, sq, kc, sk, vc, sv = c
    want = O.attention_codes(qc, sq, kc, sk, vc, sv, scale)
    P = O.attention_probs(qc, sq, kc, sk, scale)
    return want, AB.attention_bound(want, P, qc, sq, kc, sk, vc, sv, scale)


SHAPES = [(1, 300, 4097, 128), (4, 129, 129, 64), (2, 130, 200, 64), (1, 128, 1000, 128)]


@pytest.mark.parametrize("BH,Lq,Lk,D", SHAPES)
def test_kernel_model_inside_bound(O, BH, Lq, Lk, D):
    c = _case(O, BH, Lq, Lk, D, BH * 1000 + Lq + Lk + D)
    scale = 1.0 / np.sqrt(D)
    want, bound = _bound(O, c, scale)
    model = AB.kernel_model(*c, scale)
    assert np.all(np.abs(model - want) <= bound)


def test_kernel_model_peaky_softmax(O):
    c = _case(O, 1, 200, 333, 128, 42, qscale=4.0)
    want, bound = _bound(O, c, 0.5)
    assert np.all(np.abs(AB.kernel_model(*c, 0.5) - want) <= bound)


@pytest.mark.parametrize("BH,Lq,Lk,D", [(1, 300, 4097, 128), (4, 129, 129, 64)])
def test_dropped_keys_fall_outside(O, BH, Lq, Lk, D):
    qc, sq, kc, sk, vc, sv = c = _case(O, BH, Lq, Lk, D, BH * 1000 + Lq + Lk + D)
    scale = 1.0 / np.sqrt(D)
    want, bound = _bound(O, c, scale)
    drop_last = np.arange(Lk - 1)
    drop_block = np.r_[0:64, 128:Lk]            # keys 64 .. 127 missing
    for keep, what in ((drop_last, "last key"), (drop_block, "one 64-key block")):
        wrong = O.attention_codes(qc, sq, kc[:, keep], sk[:, keep], vc[:, keep], sv[:, keep], scale)
        assert np.any(np.abs(wrong - want) > bound), f"dropping the {what} stays inside the bound"


def test_bound_is_tight_on_long_sequences(O):
    c = _case(O, 1, 300, 4097, 128, 1000 + 300 + 4097 + 128)
    want, bound = _bound(O, c, 1.0 / np.sqrt(128))
    assert np.median(bound / np.abs(want)) <= 0.25
