"""Pins of the oracle's routing options: scoring function, grouped top-k, score-correction bias
and routed scaling factor (experts_int8 page, ExpertsInt8MoEMethod.apply -> select_experts;
moe_wna16 page, MoeWNA16Method.apply_monolithic)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    return json.load(open(os.path.join(GOLD, "route_grouped_handworked.json")))["cases"]


def _run(c, **over):
    a = dict(k=c["k"], renormalize=c["renormalize"], scoring=c["scoring"], num_expert_group=c["num_expert_group"],
             topk_group=c["topk_group"], bias=None if c["bias"] is None else np.array(c["bias"], np.float32),
             routed_scaling_factor=c["routed_scaling_factor"])
    a.update(over)
    return oracle.route_select(np.array(c["logits"], np.float32), **a)


@pytest.mark.parametrize("i", range(4))
def test_handworked(i):
    c = _cases()[i]
    w, ids = _run(c)
    np.testing.assert_array_equal(ids, np.array(c["ids"], np.int32))
    np.testing.assert_allclose(w, np.array(c["weights"]), rtol=1e-12, atol=0)


def test_handworked_contrasts():
    """The options matter: without groups / without the bias the golden cases pick other experts."""
    a, b = _cases()[0], _cases()[1]
    _, ids = _run(a, num_expert_group=0, topk_group=0)
    np.testing.assert_array_equal(ids, np.array(a["ungrouped_ids"]))
    _, ids = _run(b, bias=None)
    np.testing.assert_array_equal(ids, np.array(b["unbiased_ids"]))


def test_defaults_equal_the_softmax_router():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 16)).astype(np.float32)
    l[3, 5] = l[3, 9]                                      # a tie
    for k in (1, 2, 6):
        for renorm in (True, False):
            w0, i0 = oracle.route_softmax_topk(l, k, renorm)
            w1, i1 = oracle.route_select(l, k, renorm)
            np.testing.assert_array_equal(i0, i1)
            np.testing.assert_allclose(w0, w1, rtol=1e-15)


def test_sigmoid_weights_are_sigmoid_and_order_by_logit():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((20, 12)).astype(np.float32)
    w, ids = oracle.route_select(l, 3, renormalize=False, scoring="sigmoid")
    _, ids_soft = oracle.route_softmax_topk(l, 3)
    np.testing.assert_array_equal(ids, ids_soft)           # both scores increase with the logit
    sig = torch.sigmoid(torch.from_numpy(l.astype(np.float64))).numpy()
    np.testing.assert_allclose(w, np.take_along_axis(sig, ids.astype(np.int64), 1), rtol=1e-15)


def test_one_group_and_all_groups_change_nothing():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((30, 16)).astype(np.float32)
    b = (0.3 * rng.standard_normal(16)).astype(np.float32)
    ref = oracle.route_select(l, 4, True, "sigmoid", bias=b)
    for G, tg in ((1, 1), (4, 4), (16, 16)):
        got = oracle.route_select(l, 4, True, "sigmoid", num_expert_group=G, topk_group=tg, bias=b)
        np.testing.assert_array_equal(got[1], ref[1])
        np.testing.assert_array_equal(got[0], ref[0])


def test_scaling_factor_is_linear():
    rng = np.random.default_rng(6)
    l = rng.standard_normal((10, 8)).astype(np.float32)
    w1, i1 = oracle.route_select(l, 2, True, "sigmoid")
    w2, i2 = oracle.route_select(l, 2, True, "sigmoid", routed_scaling_factor=2.5)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_allclose(w2, 2.5 * w1, rtol=1e-15)
    np.testing.assert_allclose(w1.sum(1), 1.0, rtol=1e-14)


def _bruteforce(key, k, G, tg):
    """All (groups, experts) choices consistent with the definition, by enumeration (tiny E)."""
    E = key.size
    gs = E // G
    gkey = [max(key[g * gs:(g + 1) * gs]) for g in range(G)]
    best = []
    for groups in itertools.combinations(range(G), tg):
        rest = [g for g in range(G) if g not in groups]
        if not all(gkey[a] >= gkey[r] for a in groups for r in rest):
            continue
        cand = [e for g in groups for e in range(g * gs, (g + 1) * gs)]
        for sub in itertools.combinations(cand, k):
            others = [e for e in cand if e not in sub]
            if all(key[a] >= key[o] for a in sub for o in others):
                best.append(set(sub))
    return best


def test_grouped_against_bruteforce():
    rng = np.random.default_rng(7)
    for trial in range(60):
        E, G = 8, (2, 4)[trial % 2]
        tg = 1 + trial % G
        k = 1 + trial % min(3, tg * (E // G))
        l = rng.integers(-3, 4, size=(1, E)).astype(np.float32)     # many ties on purpose
        b = rng.integers(-2, 3, size=E).astype(np.float32) * 0.125 if trial % 3 else None
        _, ids = oracle.route_select(l, k, True, "sigmoid", G, tg, b)
        key = l[0]
        if b is not None:
            s = (1 / (1 + np.exp(-l[0].astype(np.float64)))).astype(np.float32)
            key = (s + b).astype(np.float32)
        assert set(ids[0].tolist()) in _bruteforce(key, k, G, tg), (l, b, ids)
        kk = key[ids[0]]
        assert np.all(kk[:-1] >= kk[1:])                                # descending


def test_bad_group_arguments():
    l = np.zeros((1, 8), np.float32)
    with pytest.raises(ValueError):
        oracle.route_select(l, 2, num_expert_group=3, topk_group=1)     # 8 does not split in 3
    with pytest.raises(ValueError):
        oracle.route_select(l, 5, num_expert_group=4, topk_group=2)     # only 4 experts kept
    with pytest.raises(ValueError):
        oracle.route_select(l, 2, scoring="tanh")
