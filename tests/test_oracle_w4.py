"""Pins of the oracle's group-wise W4 path (moe_wna16 page: create_weights, weight loader zero convention)."""
import json
import os

import numpy as np
import pytest

import oracle
from weight_quantized_mixture_amd import synthetic

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_handworked_group():
    g = json.load(open(os.path.join(GOLD, "w4_handworked.json")))
    w = np.array([g["w"]], np.float32)
    q, s, z = oracle.quantize_w4_groups(w, g["group_size"])
    assert float(s[0, 0]) == g["scale_fp16"]
    assert int(z[0, 0]) == g["zero"]
    np.testing.assert_array_equal(q[0], g["q"])
    packed = oracle.pack_w4_along_k(q)
    assert packed.shape == (1, 1)
    assert format(int(packed.view(np.uint32)[0, 0]), "08X") == g["packed_word_hex"]
    zp = oracle.pack_w4_along_n(np.repeat(z, 8, axis=0))
    W = oracle.dequant_w4(np.repeat(packed, 8, axis=0), np.repeat(s, 8, axis=0), zp, g["group_size"])
    np.testing.assert_array_equal(W[0], g["dequant"])


def test_pack_roundtrip_bruteforce():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 16, size=(3, 16, 64)).astype(np.uint8)
    p = oracle.pack_w4_along_k(q)
    assert p.dtype == np.int32 and p.shape == (3, 16, 8)
    np.testing.assert_array_equal(oracle.unpack_w4_along_k(p), q)
    # brute force: element k of row n sits at bits 4*(k%8) of word k//8
    for n in range(16):
        for kk in range(64):
            word = int(p.view(np.uint32)[1, n, kk // 8])
            assert (word >> (4 * (kk % 8))) & 0xF == q[1, n, kk]
    z = rng.integers(0, 16, size=(2, 24, 5)).astype(np.uint8)
    pz = oracle.pack_w4_along_n(z)
    assert pz.shape == (2, 3, 5)
    np.testing.assert_array_equal(oracle.unpack_w4_along_n(pz), z)
    for n in range(24):
        for gi in range(5):
            assert (int(pz.view(np.uint32)[0, n // 8, gi]) >> (4 * (n % 8))) & 0xF == z[0, n, gi]


def test_canonical_uint8_bytes_match_int32_words():
    # the page's canonical layout keeps two codes per byte along K, the even code in the low nibble;
    # read as little-endian int32 it is the same bytes as this packing
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, size=(4, 32)).astype(np.uint8)
    canon = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.pack_w4_along_k(q).view(np.uint8), canon)


@pytest.mark.parametrize("g", [32, 128])
def test_quantizer_invariants(g):
    w = synthetic.random_master((2, 16, 256), 3)
    q, s, z = oracle.quantize_w4_groups(w, g)
    assert q.max() <= 15 and z.max() <= 15
    W = np.stack([oracle.dequant_w4(oracle.pack_w4_along_k(q[e]), s[e], oracle.pack_w4_along_n(z[e]), g)
                  for e in range(2)])
    sk = np.repeat(s.astype(np.float64), g, axis=-1)
    # N(0, 0.02) data never clips, so the error is at most half a step plus the fp16 rounding of the scale
    err = np.abs(W - w)
    assert np.all(err <= sk * 0.5 + 15 * sk * 2.0 ** -11 + 1e-12)


def test_w4_forward_equals_dense_forward():
    E, k, H, I, T, g = 4, 2, 64, 32, 5, 32
    w13 = synthetic.random_master((E, 2 * I, H), 8, tag=50)
    w2 = synthetic.random_master((E, H, I), 8, tag=51)
    q13, s13, z13 = oracle.quantize_w4_groups(w13, g)
    q2, s2, z2 = oracle.quantize_w4_groups(w2, g)
    P13, Z13 = oracle.pack_w4_along_k(q13), np.stack([oracle.pack_w4_along_n(z13[e]) for e in range(E)])
    P2, Z2 = oracle.pack_w4_along_k(q2), np.stack([oracle.pack_w4_along_n(z2[e]) for e in range(E)])
    x = oracle.fp16_bits_to_f64(synthetic.random_activations(T, H, "fp16", 8))
    w, ids = oracle.route_softmax_topk(synthetic.random_logits(T, E, 8), k, True)
    out = oracle.moe_forward_w4(x, P13, s13, Z13, P2, s2, Z2, g, w, ids)
    D13 = (q13.astype(np.float64) - np.repeat(z13, g, -1)) * np.repeat(s13.astype(np.float64), g, -1)
    D2 = (q2.astype(np.float64) - np.repeat(z2, g, -1)) * np.repeat(s2.astype(np.float64), g, -1)
    ref = oracle.moe_forward_dense(x, lambda e: D13[e], lambda e: D2[e], w, ids, I)
    np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-16)
    # options: shared expert (the last one) and the routing weight on the input
    ids_r = np.where(ids < E - 1, ids, 0).astype(np.int32)
    for woi in (False, True):
        out = oracle.moe_forward_w4(x, P13, s13, Z13, P2, s2, Z2, g, w, ids_r, weight_on_input=woi, num_shared=1)
        we, ie = oracle.with_shared_experts(w, ids_r, E - 1, 1)
        ref = oracle.moe_forward_dense(x, lambda e: D13[e], lambda e: D2[e], we, ie, I, weight_on_input=woi)
        np.testing.assert_allclose(out, ref, rtol=1e-14, atol=1e-16)
        if woi:
            we[:, -1] = 1.0
            ref2 = oracle.moe_forward_dense(x, lambda e: D13[e], lambda e: D2[e], we, ie, I, weight_on_input=True)
            np.testing.assert_allclose(out, ref2, rtol=1e-14, atol=1e-16)
