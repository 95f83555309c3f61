"""Pins of the oracle's layer forward (experts_int8 page: create_weights, quantizing_weight_loader, apply)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from weight_quantized_mixture_amd import synthetic

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _tiny_layer(E=4, k=2, H=32, I=24, T=9, seed=0):
    q13, s13 = oracle.quantize_int8_rows(synthetic.random_master((E, 2 * I, H), seed, tag=40))
    q2, s2 = oracle.quantize_int8_rows(synthetic.random_master((E, H, I), seed, tag=41))
    x = oracle.bf16_bits_to_f64(synthetic.random_activations(T, H, "bf16", seed))
    l = synthetic.random_logits(T, E, seed)
    w, ids = oracle.route_softmax_topk(l, k, True)
    return x, q13, s13, q2, s2, w, ids


def test_handworked_layer():
    g = json.load(open(os.path.join(GOLD, "layer_handworked.json")))
    out = oracle.moe_forward_w8(np.array(g["x"]), np.array(g["q13"], np.int8), np.array(g["s13"], np.float32),
                                np.array(g["q2"], np.int8), np.array(g["s2"], np.float32),
                                np.array(g["topk_w"]), np.array(g["topk_ids"]))
    np.testing.assert_allclose(out, g["out"], rtol=1e-15, atol=1e-16)


def test_dense_masked_sum_equals_routed():
    x, q13, s13, q2, s2, w, ids = _tiny_layer()
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    T, H = x.shape
    E, I = q13.shape[0], q13.shape[1] // 2
    dense = np.zeros_like(out)
    for t in range(T):                  # every token through every expert, weight 0 if unrouted
        for e in range(E):
            m = sum(w[t, j] for j in range(ids.shape[1]) if ids[t, j] == e)
            W13 = q13[e].astype(np.float64) * s13[e][:, None]
            W2 = q2[e].astype(np.float64) * s2[e][:, None]
            hvec = W13 @ x[t]
            gate, up = hvec[:I], hvec[I:]
            a = gate / (1 + np.exp(-gate)) * up
            dense[t] += m * (W2 @ a)
    np.testing.assert_allclose(out, dense, rtol=1e-12, atol=1e-15)


def test_single_expert_top1_is_gated_mlp():
    E, H, I, T = 1, 48, 40, 7
    q13, s13 = oracle.quantize_int8_rows(synthetic.random_master((E, 2 * I, H), 3, tag=42))
    q2, s2 = oracle.quantize_int8_rows(synthetic.random_master((E, H, I), 3, tag=43))
    x = oracle.bf16_bits_to_f64(synthetic.random_activations(T, H, "bf16", 3))
    w, ids = oracle.route_softmax_topk(synthetic.random_logits(T, E, 3), 1, True)
    assert np.all(w == 1.0) and np.all(ids == 0)
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    W1 = torch.from_numpy(q13[0, :I].astype(np.float64) * s13[0, :I, None])     # gate_proj
    W3 = torch.from_numpy(q13[0, I:].astype(np.float64) * s13[0, I:, None])     # up_proj
    W2 = torch.from_numpy(q2[0].astype(np.float64) * s2[0, :, None])            # down_proj
    X = torch.from_numpy(x)
    ref = (torch.nn.functional.silu(X @ W1.T) * (X @ W3.T)) @ W2.T
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-15)


def test_token_permutation_and_expert_relabel():
    x, q13, s13, q2, s2, w, ids = _tiny_layer(seed=2)
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    perm = np.random.default_rng(0).permutation(x.shape[0])
    out_p = oracle.moe_forward_w8(x[perm], q13, s13, q2, s2, w[perm], ids[perm])
    np.testing.assert_allclose(out_p, out[perm], rtol=1e-13, atol=1e-16)
    E = q13.shape[0]
    lab = np.random.default_rng(1).permutation(E)          # expert e is stored at slot lab[e]
    inv = np.argsort(lab)
    out_r = oracle.moe_forward_w8(x, q13[inv], s13[inv], q2[inv], s2[inv], w, lab[ids])
    np.testing.assert_allclose(out_r, out, rtol=1e-13, atol=1e-16)


def test_linear_in_w2_scale_and_weights():
    x, q13, s13, q2, s2, w, ids = _tiny_layer(seed=4)
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    out2 = oracle.moe_forward_w8(x, q13, s13, q2, (2 * s2).astype(np.float32), w, ids)
    np.testing.assert_allclose(out2, 2 * out, rtol=1e-14, atol=0)
    # one token's weight set to zero removes that term only
    w0 = w.copy(); w0[0, 1] = 0
    out3 = oracle.moe_forward_w8(x, q13, s13, q2, s2, w0, ids)
    np.testing.assert_allclose(out3[1:], out[1:], rtol=0, atol=0)


def test_gate_up_order_matters():
    # swapping the gate and up halves (a plausible mistake) changes the result
    x, q13, s13, q2, s2, w, ids = _tiny_layer(seed=5)
    I = q13.shape[1] // 2
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    sw = np.concatenate([q13[:, I:], q13[:, :I]], axis=1)
    ss = np.concatenate([s13[:, I:], s13[:, :I]], axis=1)
    out_sw = oracle.moe_forward_w8(x, sw, ss, q2, s2, w, ids)
    assert np.abs(out_sw - out).max() > 1e-3 * np.abs(out).max()


def test_out_of_range_ids_contribute_nothing():
    x, q13, s13, q2, s2, w, ids = _tiny_layer(seed=6)
    ids2 = ids.copy(); ids2[3, 1] = 99; ids2[4, 0] = -1
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    out2 = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids2)
    np.testing.assert_array_equal(out2[:3], out[:3])
    ref = oracle.moe_forward_w8(x[3:5], q13, s13, q2, s2, np.array([[w[3, 0], 0.0], [0.0, w[4, 1]]]),
                                np.array([[ids[3, 0], ids[3, 0]], [ids[4, 1], ids[4, 1]]]))
    np.testing.assert_allclose(out2[3:5], ref, rtol=1e-14, atol=1e-16)


def test_tolerance_helper():
    ref = np.array([1.0, -2.0, 0.0, 1e-5])
    ok, _ = oracle.layer_within_tolerance(ref + np.array([0.019, 0.03, 0.0009, 0.0]), ref)
    assert ok
    ok, d = oracle.layer_within_tolerance(ref + np.array([0.0, 0.0, 0.0011, 0.0]), ref)
    assert not ok and d["n_bad"] == 1


def _golden():
    g = json.load(open(os.path.join(GOLD, "layer_handworked.json")))
    return g, np.array(g["x"]), np.array(g["q13"], np.int8), np.array(g["s13"], np.float32), \
        np.array(g["q2"], np.int8), np.array(g["s2"], np.float32)


def test_weight_on_input_handworked():
    """experts_int8 page, apply(apply_router_weight_on_input): the weight scales the expert input."""
    g, x, q13, s13, q2, s2 = _golden()
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, np.array(g["topk_w"]), np.array(g["topk_ids"]),
                                weight_on_input=True)
    np.testing.assert_allclose(out, g["weight_on_input"]["out"], rtol=1e-15, atol=1e-16)


def test_shared_experts_handworked():
    """moe_wna16 page, MoeWNA16Method.apply(shared_experts): shared experts added for every token."""
    g, x, q13, s13, q2, s2 = _golden()
    sh = g["shared"]
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, np.array(sh["topk_w"]), np.array(sh["topk_ids"]),
                                num_shared=sh["num_shared"])
    np.testing.assert_allclose(out, sh["out"], rtol=1e-15, atol=1e-16)


def test_weight_on_input_is_the_scaled_input_through_a_gated_mlp():
    x, q13, s13, q2, s2, w, ids = _tiny_layer(seed=8)
    ones = np.ones_like(w)
    np.testing.assert_allclose(oracle.moe_forward_w8(x, q13, s13, q2, s2, ones, ids, weight_on_input=True),
                               oracle.moe_forward_w8(x, q13, s13, q2, s2, ones, ids), rtol=1e-14, atol=1e-16)
    # token by token: sum_j MLP_e(w x) with torch's silu on the dequantized expert
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids, weight_on_input=True)
    I = q13.shape[1] // 2
    for t in range(x.shape[0]):
        acc = torch.zeros(x.shape[1], dtype=torch.float64)
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            W1 = torch.from_numpy(q13[e, :I].astype(np.float64) * s13[e, :I, None])
            W3 = torch.from_numpy(q13[e, I:].astype(np.float64) * s13[e, I:, None])
            W2 = torch.from_numpy(q2[e].astype(np.float64) * s2[e, :, None])
            xi = torch.from_numpy(w[t, j] * x[t])
            acc += (torch.nn.functional.silu(W1 @ xi) * (W3 @ xi)) @ W2.T
        np.testing.assert_allclose(out[t], acc.numpy(), rtol=1e-12, atol=1e-15)
    # the weight is not linear through the layer: scaling the output instead differs
    assert np.abs(out - oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)).max() > 1e-4 * np.abs(out).max()


def test_shared_experts_add_a_gated_mlp_for_every_token():
    x, q13, s13, q2, s2, w, ids = _tiny_layer(E=5, seed=9)
    E_routed = 4
    ids = np.where(ids < E_routed, ids, 0).astype(np.int32)
    routed = oracle.moe_forward_w8(x, q13[:E_routed], s13[:E_routed], q2[:E_routed], s2[:E_routed], w, ids)
    out = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids, num_shared=1)
    I = q13.shape[1] // 2
    W1 = torch.from_numpy(q13[4, :I].astype(np.float64) * s13[4, :I, None])
    W3 = torch.from_numpy(q13[4, I:].astype(np.float64) * s13[4, I:, None])
    W2 = torch.from_numpy(q2[4].astype(np.float64) * s2[4, :, None])
    X = torch.from_numpy(x)
    shared = ((torch.nn.functional.silu(X @ W1.T) * (X @ W3.T)) @ W2.T).numpy()
    np.testing.assert_allclose(out, routed + shared, rtol=1e-12, atol=1e-15)
    # with weight on input the shared expert still takes the unscaled input
    out_i = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids, weight_on_input=True, num_shared=1)
    routed_i = oracle.moe_forward_w8(x, q13[:E_routed], s13[:E_routed], q2[:E_routed], s2[:E_routed], w, ids,
                                     weight_on_input=True)
    np.testing.assert_allclose(out_i, routed_i + shared, rtol=1e-12, atol=1e-15)


def test_combine_handworked():
    g = json.load(open(os.path.join(GOLD, "combine_handworked.json")))
    out = oracle.combine_topk(np.array(g["y_parts"]), np.array(g["topk_w"]), np.array(g["topk_ids"]), g["E"])
    np.testing.assert_array_equal(out, np.array(g["out"]))


def test_combine_of_expert_outputs_equals_layer():
    # the per-assignment expert outputs, split into three parts (two random
    # ones and the remainder), combine to the layer's output
    x, q13, s13, q2, s2, w, ids = _tiny_layer(E=5, k=3, T=7, seed=3)
    E, I = q13.shape[0], q13.shape[1] // 2
    ids = ids.copy()
    ids[2, 1] = -1                      # a dropped assignment
    ids[4, 0] = E                       # an id past the experts
    T, k = ids.shape
    y = np.zeros((T * k, x.shape[1]))
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                a = oracle.moe_expert_intermediate(x[t][None], oracle.dequant_int8_rows(q13[e], s13[e]), I)[0]
                y[t * k + j] = oracle.dequant_int8_rows(q2[e], s2[e]) @ a
    rng = np.random.default_rng(5)
    r1, r2 = rng.standard_normal(y.shape), rng.standard_normal(y.shape)
    parts = np.stack([y - r1 - r2, r1, r2])
    got = oracle.combine_topk(parts, w, ids, E)
    ref = oracle.moe_forward_w8(x, q13, s13, q2, s2, w, ids)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the flat index is t*k + j: a transposed (j*T + t) reading fails
    bad = oracle.combine_topk(parts.reshape(3, T, k, -1).transpose(0, 2, 1, 3).reshape(3, T * k, -1), w, ids, E)
    assert not np.allclose(bad, ref, rtol=1e-6)
