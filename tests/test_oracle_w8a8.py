"""Pins of the oracle's W8A8 layer (fused_moe oracle/int8 page, select_int8_moe_backend:
per-channel int8 weights, dynamic per-token int8 activations)."""
import json
import os

import numpy as np

import oracle
from weight_quantized_mixture_amd import synthetic

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _g():
    return json.load(open(os.path.join(GOLD, "w8a8_handworked.json")))


def test_activation_codes_handworked():
    g = _g()
    q, s = oracle.quantize_act_int8_rows(np.array(g["x"]))
    np.testing.assert_array_equal(q, g["x_codes"])
    np.testing.assert_array_equal(s, g["x_scales"])
    for r in g["rows"]:
        q, s = oracle.quantize_act_int8_rows(np.array([r["a"]]))
        np.testing.assert_array_equal(q[0], r["a_codes"])
        assert float(s[0]) == r["a_scale"]


def test_layer_handworked():
    g = _g()
    out = oracle.moe_forward_w8a8(np.array(g["x"]), np.array(g["q13"], np.int8), np.array(g["s13"], np.float32),
                                  np.array(g["q2"], np.int8), np.array(g["s2"], np.float32), np.ones((2, 1)),
                                  np.zeros((2, 1), np.int32))
    np.testing.assert_allclose(out, g["out"], rtol=1e-12, atol=0)


def _layer(E=4, k=2, H=32, I=24, T=9, seed=0):
    q13, s13 = oracle.quantize_int8_rows(synthetic.random_master((E, 2 * I, H), seed, tag=40))
    q2, s2 = oracle.quantize_int8_rows(synthetic.random_master((E, H, I), seed, tag=41))
    x = oracle.bf16_bits_to_f64(synthetic.random_activations(T, H, "bf16", seed))
    w, ids = oracle.route_softmax_topk(synthetic.random_logits(T, E, seed), k, True)
    return x, q13, s13, q2, s2, w, ids


def test_close_to_w8a16_within_the_quantization_bound():
    """Each activation code is within half a step of its value, so the W8A8 output stays within the
    bound those half steps allow around the exact (W8A16) layer."""
    x, q13, s13, q2, s2, w, ids = _layer(seed=3)
    got = oracle.moe_forward_w8a8(x, q13, s13, q2, s2, w, ids)
    ref = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert 1e-5 < rel < 5e-2, rel                     # quantized, but close


def test_integer_inputs_make_gemm1_exact():
    """With x rows whose largest magnitude is 127 and integer entries, the codes are x itself (scale 1),
    so GEMM1 and the intermediate equal the W8A16 ones exactly."""
    x, q13, s13, q2, s2, w, ids = _layer(seed=4)
    xi = np.rint(x * 40).clip(-127, 127)
    xi[:, 0] = 127.0
    qx, sx = oracle.quantize_act_int8_rows(xi)
    np.testing.assert_array_equal(qx, xi)
    assert np.all(sx == 1.0)
    I = q13.shape[1] // 2
    for e in range(q13.shape[0]):
        W13 = oracle.dequant_int8_rows(q13[e], s13[e])
        h8 = (qx.astype(np.int64) @ q13[e].astype(np.int64).T) * s13[e].astype(np.float64)
        np.testing.assert_allclose(oracle.silu(h8[:, :I]) * h8[:, I:], oracle.moe_expert_intermediate(xi, W13, I),
                                   rtol=1e-13, atol=1e-15)


def test_dense_masked_sum_and_options():
    x, q13, s13, q2, s2, w, ids = _layer(seed=5)
    out = oracle.moe_forward_w8a8(x, q13, s13, q2, s2, w, ids)
    dense = np.zeros_like(out)
    for t in range(x.shape[0]):
        for e in range(q13.shape[0]):
            m = sum(w[t, j] for j in range(ids.shape[1]) if ids[t, j] == e)
            if m:
                dense[t] += m * oracle.moe_forward_w8a8(x[t:t + 1], q13, s13, q2, s2, np.ones((1, 1)),
                                                        np.array([[e]], np.int32))[0]
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-15)
    # zero rows quantize to zero and contribute nothing
    x0 = x.copy(); x0[2] = 0
    assert np.all(oracle.moe_forward_w8a8(x0, q13, s13, q2, s2, w, ids)[2] == 0)
    # shared expert: routed + the shared expert's own W8A8 output with weight 1
    E = q13.shape[0]
    ids_r = np.where(ids < E - 1, ids, 0).astype(np.int32)
    both = oracle.moe_forward_w8a8(x, q13, s13, q2, s2, w, ids_r, num_shared=1)
    routed = oracle.moe_forward_w8a8(x, q13[:E - 1], s13[:E - 1], q2[:E - 1], s2[:E - 1], w, ids_r)
    shared = oracle.moe_forward_w8a8(x, q13, s13, q2, s2, np.ones((x.shape[0], 1)),
                                     np.full((x.shape[0], 1), E - 1, np.int32))
    np.testing.assert_allclose(both, routed + shared, rtol=1e-12, atol=1e-15)


def test_intermediate_scales():
    """The scales the W8A8 forward quantizes its intermediate with: y of one assignment is
    sa * s2 * (q2 a8), so a routed token's output equals the sum over its assignments."""
    g = _g()
    sa = oracle.moe_w8a8_intermediate_scales(np.array(g["x"]), np.array(g["q13"], np.int8),
                                             np.array(g["s13"], np.float32), np.ones((2, 1)),
                                             np.zeros((2, 1), np.int32))
    np.testing.assert_array_equal(sa[:, 0], [r["a_scale"] for r in g["rows"]])
    x, q13, s13, q2, s2, w, ids = _layer(seed=8)
    ids2 = ids.copy(); ids2[0, 1] = -1
    sa = oracle.moe_w8a8_intermediate_scales(x, q13, s13, w, ids2)
    assert sa[0, 1] == 0 and np.all(sa[1:] > 0)
