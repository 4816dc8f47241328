"""Pins of the chunk path's precision model (tests/chunk_model.py) on the CPU.

The model applies the chunk path's documented roundings (bf16 weights formed
as the fp32 sum (c1 + c2) + c3, bf16 tokens, bf16 h) around float64 products.
It is checked against the fp64 oracle: exactly where every rounding is exact,
and within the rounding error budget elsewhere.
"""
import numpy as np
import pytest

import chunk_model as M
from oracle import oracle as O
from synth import synth as S


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1)
    assert M.bf16(np.float32(1.0 + 2.0 ** -8))[()] == 1.0
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert M.bf16(np.float32(1.0 + 3 * 2.0 ** -8))[()] == 1.0 + 2.0 ** -6
    assert M.bf16(np.float32(1.0 + 2.0 ** -8 + 2.0 ** -20))[()] == 1.0 + 2.0 ** -7
    assert M.bf16(np.float32(-3.0))[()] == -3.0
    rng = np.random.default_rng(0)
    v = rng.standard_normal(10000).astype(np.float32)
    r = M.bf16(v)
    assert np.all(np.abs(r - v) <= np.abs(v) * 2.0 ** -8)       # within half an ulp (8 significant bits)
    assert np.all((r.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)


def test_model_is_exact_where_every_rounding_is_exact():
    """Small-integer tokens and one-hot stage codebooks scaled by 1, 2, 4 make
    every weight an integer in [-7, 7]: tokens, weights, a and b are exact, so
    the model's pre-activations equal the oracle's, and its output equals the
    oracle's down projection of bf16(h) (up to fp64 summation order)."""
    d, ffn = 64, 48
    rng = np.random.default_rng(1)
    cb = np.zeros((3, 3, 256, 8), np.float32)
    for m, signs in enumerate([(1, 2, 4), (1, -2, 4), (-1, 2, 4)]):
        for s in range(3):
            cb[m, s, np.arange(256), np.arange(256) % 8] = signs[s]
    rec = rng.integers(0, 256, S.record_bytes(d, ffn), dtype=np.uint8)
    x = rng.integers(-3, 4, d).astype(np.float32)
    y, Wd, H = M.expert(cb, rec, d, ffn, M.token_x(x, False, 0.0))
    ref = O.expert(d, ffn, cb, rec, x.astype(np.float64))
    gc, uc, dc = M.matrices(rec, d, ffn)
    a = M.dense_weights(cb[0], gc) @ x
    assert np.array_equal(a, ref.pre_gate)
    assert np.array_equal(M.dense_weights(cb[1], uc) @ x, ref.pre_up)
    assert np.array_equal(H, M.bf16(ref.h.astype(np.float32)))
    # the last product sums bf16 values of mixed magnitude: fp64 summation order only
    np.testing.assert_allclose(y, O.matvec(cb[2], dc, H), rtol=1e-13, atol=0)


@pytest.mark.parametrize("shape", [S.TINY, S.Shape(264, 136, 5, 2, "f16")])
def test_model_within_bf16_budget_of_the_oracle(shape):
    """Random synthetic layers: the model's output is within 2e-2 relative L2
    of the fp64 oracle (the chunk path's bar) and within a few bf16 ulps in
    total; its per-element scales bound its own deviation from the oracle."""
    cb = S.codebooks(4, 0, shape.n_experts, shape.np_cb_dtype)
    w_r = S.router_weights(4, 0, shape.d, shape.n_experts)
    bank = S.codes_bank(4, 0, shape.n_experts, shape.record_bytes)
    xs = S.tokens(4, 0, 6, shape.d)
    for x in xs:
        ref = O.layer(x, w_r, shape.top_k, lambda e: cb[e], lambda e: bank[e], shape.d, shape.ffn)
        y, peak, mass = M.layer(x, ref.route.ids, ref.route.gates, lambda e: cb[e], lambda e: bank[e],
                                shape.d, shape.ffn)
        err = np.linalg.norm(y - ref.delta) / np.linalg.norm(ref.delta)
        assert 1e-5 < err < 2e-2, err   # really rounded, and within the bar
        # model vs fp64 at first order: weights, tokens and h each within 2^-9
        # relative, propagated through both products (a loose element bound)
        assert np.all(np.abs(y - ref.delta) <= 2.0 ** -5 * mass + 1e-12)
