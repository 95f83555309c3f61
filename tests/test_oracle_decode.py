"""Pins of the oracle's activation decoding and its per-expert intermediate.

* bf16 / fp16 decoding (experts_int8 page, ExpertsInt8Config.get_supported_act_dtypes:
  bfloat16 and float16 activations): hand-decoded IEEE bit patterns in
  tests/golden/act_decode_handworked.json, exact.
* moe_expert_intermediate (experts_int8 page, apply: activation "silu" on the
  gate rows times the up rows of w13): the hand-worked layer's intermediate
  values in tests/golden/layer_handworked.json.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cases(kind):
    g = json.load(open(os.path.join(GOLD, "act_decode_handworked.json")))
    bits = np.array([int(c["bits"], 16) for c in g[kind]], np.uint16)
    vals = np.array([float.fromhex(c["value"]) for c in g[kind]], np.float64)
    return bits, vals


def _same(got, want):
    # exact, including the sign of zero
    return np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))


@pytest.mark.parametrize("kind,fn", [("bf16", oracle.bf16_bits_to_f64), ("fp16", oracle.fp16_bits_to_f64)])
def test_decode_handworked(kind, fn):
    bits, vals = _cases(kind)
    got = fn(bits)
    assert got.dtype == np.float64
    assert _same(got, vals), (got, vals)
    assert _same(oracle.act_bits_to_f64(bits, kind), vals)


def test_decode_dispatch_and_shape():
    bits, vals = _cases("bf16")
    b2 = np.stack([bits, bits[::-1]])
    got = oracle.act_bits_to_f64(b2, "bf16")
    assert got.shape == b2.shape
    assert _same(got[1], vals[::-1])
    with pytest.raises(ValueError):
        oracle.act_bits_to_f64(bits, "fp8")


def test_decode_pins_catch_plausible_mistakes():
    """A decode with a wrong shift, the wrong format, or a dropped sign fails the golden."""
    bits, vals = _cases("bf16")
    wrong_shift = (bits.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
    assert not _same(wrong_shift, vals)
    assert not _same(oracle.fp16_bits_to_f64(bits), vals)          # fp16 read of bf16 bits
    hb, hv = _cases("fp16")
    assert not _same(oracle.bf16_bits_to_f64(hb), hv)              # bf16 read of fp16 bits
    no_sign = np.abs(oracle.bf16_bits_to_f64(bits))
    assert not _same(no_sign, vals)


def _golden_layer():
    g = json.load(open(os.path.join(GOLD, "layer_handworked.json")))
    x = np.array(g["x"], np.float64)
    q13 = np.array(g["q13"], np.int8)
    s13 = np.array(g["s13"], np.float32)
    return g, x, q13, s13


def test_intermediate_handworked():
    g, x, q13, s13 = _golden_layer()
    I = g["I"]
    for (t, e), want in zip(g["intermediate"]["rows"], g["intermediate"]["a"]):
        W13 = oracle.dequant_int8_rows(q13[e], s13[e])
        a = oracle.moe_expert_intermediate(x[t:t + 1], W13, I)
        assert a.shape == (1, I)
        assert math.isclose(float(a[0, 0]), want, rel_tol=1e-15, abs_tol=0.0), (t, e, a, want)


def test_intermediate_closed_forms():
    # the derivation's closed forms: 2 / (1 + e^-1) and -1 / (1 + e^0.5)
    g, *_ = _golden_layer()
    a0, a1 = g["intermediate"]["a"]
    assert math.isclose(a0, 2.0 / (1.0 + math.exp(-1.0)), rel_tol=1e-15)
    assert math.isclose(a1, -1.0 / (1.0 + math.exp(0.5)), rel_tol=1e-15)


def test_intermediate_gate_up_swap_detected():
    """Feeding the up rows as gate (a plausible mistake) changes both golden values."""
    g, x, q13, s13 = _golden_layer()
    I = g["I"]
    for (t, e), want in zip(g["intermediate"]["rows"], g["intermediate"]["a"]):
        W13 = oracle.dequant_int8_rows(q13[e], s13[e])
        swapped = np.concatenate([W13[I:], W13[:I]], axis=0)
        a = oracle.moe_expert_intermediate(x[t:t + 1], swapped, I)
        assert abs(float(a[0, 0]) - want) > 1e-3


def test_intermediate_matches_layer_with_identity_w2():
    """With W2 = identity (H = I) and weight 1, the layer output is the intermediate itself."""
    rng = np.random.default_rng(5)
    H = I = 6
    x = rng.standard_normal((3, H))
    W13 = rng.standard_normal((2 * I, H))
    a = oracle.moe_expert_intermediate(x, W13, I)
    out = oracle.moe_forward_dense(x, lambda e: W13, lambda e: np.eye(H), np.ones((3, 1)),
                                   np.zeros((3, 1), np.int32), I)
    np.testing.assert_allclose(out, a, rtol=1e-15, atol=1e-15)
