"""Pins of the oracle's GPTQ / AWQ import (moe_wna16 page, MoeWNA16Method.get_weight_loader and
create_weights): hand-worked words, round trips from codes packed by this test's own packers, the
group-size rule, and dequantization unchanged by the import."""
import json
import os

import numpy as np
import pytest

import oracle
from weight_quantized_mixture_amd import synthetic

GOLD = os.path.join(os.path.dirname(__file__), "golden")
AWQ_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)      # nibble p of an AWQ word holds column AWQ_ORDER[p]


def _g():
    return json.load(open(os.path.join(GOLD, "import_handworked.json")))


def _words(lst):
    return np.array([[int(v, 16) for v in lst]], np.uint32).view(np.int32)


def _bytes(lst):
    return np.array([[int(v, 16) for v in row] for row in lst], np.uint8)


def test_awq_handworked():
    g = _g()
    qw = _words(g["awq_qweight"]["words"]).reshape(2, 1)
    np.testing.assert_array_equal(oracle.awq_to_page_uint8(qw, "qweight"), _bytes(g["awq_qweight"]["page_uint8"]))
    qz = _words(g["awq_qzeros"]["words"]).reshape(1, 1)
    np.testing.assert_array_equal(oracle.awq_to_page_uint8(qz, "qzeros"), _bytes(g["awq_qzeros"]["page_uint8"]))


def test_gptq_zeros_handworked_and_carry():
    g = _g()
    for key in ("gptq_qzeros", "gptq_qzeros_carry"):
        qz = _words(g[key]["words"]).reshape(1, 1)
        np.testing.assert_array_equal(oracle.gptq_qzeros_to_page_uint8(qz), _bytes(g[key]["page_uint8"]))
    words = oracle.page_zeros_to_words(_bytes(g["gptq_qzeros"]["page_uint8"]))
    np.testing.assert_array_equal(words, _words(g["gptq_qzeros"]["library_words"]))


def test_group_size_rule():
    for c in _g()["group_size"]:
        if c["out"] is None:
            with pytest.raises(ValueError):
                oracle.wna16_group_size(c["H"], c["I"], c["g"])
        else:
            assert oracle.wna16_group_size(c["H"], c["I"], c["g"]) == tuple(c["out"])


# ---- the test's own packers, written from the formats' definitions ------------------------------


def pack_awq_qweight(q):            # codes [N, K] -> AWQ int32 [K, N/8] (packed along N, AWQ order)
    N, K = q.shape
    out = np.zeros((K, N // 8), np.uint32)
    for p, col in enumerate(AWQ_ORDER):
        out |= q[col::8, :].T.astype(np.uint32) << np.uint32(4 * p)
    return out.view(np.int32)


def pack_awq_qzeros(z):             # zeros [N, G] -> AWQ int32 [G, N/8]
    return pack_awq_qweight(z)


def pack_gptq_qweight(q):           # codes [N, K] -> GPTQ int32 [K/8, N] (packed along K, sequential)
    N, K = q.shape
    out = np.zeros((K // 8, N), np.uint32)
    for i in range(8):
        out |= q[:, i::8].T.astype(np.uint32) << np.uint32(4 * i)
    return out.view(np.int32)


def pack_gptq_qzeros(z):            # true zeros [N, G] in 1..15 -> GPTQ int32 [G, N/8] of zero - 1
    N, G = z.shape
    out = np.zeros((G, N // 8), np.uint32)
    for i in range(8):
        out |= (z[i::8, :].T.astype(np.uint32) - 1) << np.uint32(4 * i)
    return out.view(np.int32)


def _layer_matrix(N, K, g, seed, zmin=0):
    w = synthetic.random_master((N, K), seed, tag=80)
    q, s, z = oracle.quantize_w4_groups(w, g)
    z = np.maximum(z, zmin).astype(np.uint8)
    return q, s, z


@pytest.mark.parametrize("N,K,g", [(16, 256, 128), (64, 512, 128), (24, 384, 128)])
def test_awq_roundtrip(N, K, g):
    q, s, z = _layer_matrix(N, K, g, seed=N + K)
    qw, sc, qz = oracle.import_awq(pack_awq_qweight(q), pack_awq_qzeros(z), s.T.copy(), H=K, I=K, group_size=g)
    np.testing.assert_array_equal(qw, oracle.pack_w4_along_k(q))
    np.testing.assert_array_equal(qz, oracle.pack_w4_along_n(z))
    np.testing.assert_array_equal(sc.view(np.uint16), s.view(np.uint16))


@pytest.mark.parametrize("N,K,g", [(16, 256, 128), (64, 512, 128), (24, 384, 128)])
def test_gptq_roundtrip(N, K, g):
    q, s, z = _layer_matrix(N, K, g, seed=N * K, zmin=1)
    qw, sc, qz = oracle.import_gptq(pack_gptq_qweight(q), pack_gptq_qzeros(z), s.T.copy(), H=K, I=K, group_size=g)
    np.testing.assert_array_equal(qw, oracle.pack_w4_along_k(q))
    np.testing.assert_array_equal(qz, oracle.pack_w4_along_n(z))
    np.testing.assert_array_equal(sc.view(np.uint16), s.view(np.uint16))


def test_halved_groups_dequantize_the_same():
    """A g = 256 checkpoint of a layer with I = 1408 imports as g = 128 with every scale and zero
    repeated: the dequantized weights do not change."""
    H, I, g = 512, 1408, 256
    N, K = H, I                                      # a w2 matrix: K = I
    # I = 1408 is not a multiple of 256: build the checkpoint on 1536 columns and keep 1408 (the
    # last group is partial in the checkpoint's own layout, as it would be on disk)
    w = synthetic.random_master((N, 1536), 6, tag=81)
    q, s, z = oracle.quantize_w4_groups(w, g)
    q, s, z = q[:, :K], s[:, :(K + g - 1) // g], z[:, :(K + g - 1) // g]
    g2, f = oracle.wna16_group_size(H, I, g)
    assert (g2, f) == (128, 2)
    qw_awq = pack_awq_qweight(q)
    qz_awq = pack_awq_qzeros(z)
    qw, sc, qz = oracle.import_awq(qw_awq, qz_awq, s.T.copy(), H=H, I=I, group_size=g)
    sc, qz = sc[:, :K // g2], qz[:, :K // g2]        # repeat_interleave leaves one extra column here
    deq = oracle.dequant_w4(qw, sc, qz, g2)
    zk = np.repeat(z.astype(np.float64), g, axis=1)[:, :K]
    sk = np.repeat(s.astype(np.float64), g, axis=1)[:, :K]
    np.testing.assert_array_equal(deq, (q.astype(np.float64) - zk) * sk)


def test_import_catches_plausible_mistakes():
    q, s, z = _layer_matrix(16, 256, 128, seed=9)
    # the forward AWQ order (instead of its reverse) scrambles the columns
    b8 = pack_awq_qweight(q).view(np.uint8)
    nib = np.stack([b8 & 0xF, b8 >> 4], axis=-1).reshape(-1, 8)[:, list(AWQ_ORDER)]
    assert not np.array_equal(nib.reshape(256, 16).T, q)
    nib = np.stack([b8 & 0xF, b8 >> 4], axis=-1).reshape(-1, 8)[:, list(oracle.AWQ_REVERSE_ORDER)]
    assert np.array_equal(nib.reshape(256, 16).T, q)
    # GPTQ zeros without the +1 are off by one
    q, s, z = _layer_matrix(16, 256, 128, seed=10, zmin=1)
    assert not np.array_equal(oracle.page_zeros_to_words(np.ascontiguousarray(
        (lambda b: ((b & 0xF) + 16 * (b >> 4)).astype(np.uint8).T)(pack_gptq_qzeros(z).view(np.uint8)))),
        oracle.pack_w4_along_n(z))
