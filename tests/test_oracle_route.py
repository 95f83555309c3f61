"""Pins of the oracle's softmax top-k router (experts_int8 page, ExpertsInt8MoEMethod.apply -> select_experts)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from weight_quantized_mixture_amd import synthetic

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_handworked_cases():
    g = json.load(open(os.path.join(GOLD, "route_handworked.json")))
    for c in g["cases"]:
        w, ids = oracle.route_softmax_topk(np.array([c["logits"]], np.float32), c["k"], c["renormalize"])
        np.testing.assert_array_equal(ids[0], c["ids"])
        np.testing.assert_allclose(w[0], c["weights"], rtol=0, atol=c.get("tol", 1e-15))


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (128, 8), (5, 5)])
def test_sum_to_one_and_top1(E, k):
    l = synthetic.random_logits(40, E, seed=E + k)
    w, ids = oracle.route_softmax_topk(l, k, True)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)                    # descending probabilities
    for row in ids:
        assert len(set(row.tolist())) == k
    w1, _ = oracle.route_softmax_topk(l, 1, True)
    assert np.all(w1 == 1.0)


def test_k_equals_E_is_library_softmax_and_stable_argsort():
    l = synthetic.random_logits(16, 8, seed=3)
    l[2, 5] = l[2, 1]                                          # force a tie
    w, ids = oracle.route_softmax_topk(l, 8, False)
    ref_ids = torch.sort(-torch.from_numpy(l), dim=1, stable=True).indices.numpy()
    np.testing.assert_array_equal(ids, ref_ids)
    p = torch.softmax(torch.from_numpy(l).double(), dim=1).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(p, ids, 1), rtol=1e-14, atol=0)


def test_bruteforce_subsets():
    rng = np.random.default_rng(7)
    for trial in range(200):
        E = int(rng.integers(2, 9))
        k = int(rng.integers(1, E + 1))
        # few distinct values so ties are common
        l = rng.integers(-2, 3, size=(1, E)).astype(np.float32)
        w, ids = oracle.route_softmax_topk(l, k, True)
        subs = oracle.topk_subsets_bruteforce(l[0], k)
        assert tuple(sorted(ids[0].tolist())) in [tuple(sorted(s)) for s in subs]
        # among valid subsets the tie rule picks the lexicographically smallest sorted-by-(-l, id) list
        best = min(subs, key=lambda s: sorted(s, key=lambda e: (-l[0, e], e)))
        assert ids[0].tolist() == sorted(best, key=lambda e: (-l[0, e], e))


def test_no_renormalize_is_plain_probability():
    l = synthetic.random_logits(4, 16, seed=9)
    w, ids = oracle.route_softmax_topk(l, 4, False)
    for t in range(4):
        ex = np.exp(l[t].astype(np.float64) - l[t].max())
        np.testing.assert_allclose(w[t], ex[ids[t]] / ex.sum(), rtol=1e-14)
