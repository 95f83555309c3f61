"""GPU routing with the select_experts options (scoring, grouped top-k, correction bias, scaling
factor) against the oracle: ids bit for bit, weights within 1e-6 relative to the scaling factor."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import DEV, log

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gpu(logits, k, **opt):
    T, E = logits.shape
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    bias = opt.pop("bias", None)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(DEV)
    pkg.moe_route_select(torch.from_numpy(logits).to(DEV), k, tw, ti, e_score_correction_bias=b, **opt)
    torch.cuda.synchronize()
    return tw.cpu().numpy(), ti.cpu().numpy()


def _check(logits, k, what, **opt):
    w, ids = _gpu(logits, k, **dict(opt))
    bias = opt.pop("bias", None)
    w_ref, ids_ref = oracle.route_select(logits, k, bias=bias, **opt)
    np.testing.assert_array_equal(ids, ids_ref, err_msg=what)
    f = abs(opt.get("routed_scaling_factor", 1.0)) or 1.0
    np.testing.assert_allclose(w, w_ref, rtol=0, atol=1e-6 * f, err_msg=what)
    log(f"[route_select] {what}: ids equal, max |dw| {np.abs(w - w_ref).max():.2e}")


def test_golden_cases():
    for c in json.load(open(os.path.join(GOLD, "route_grouped_handworked.json")))["cases"]:
        _check(np.array(c["logits"], np.float32), c["k"], c["name"], renormalize=c["renormalize"],
               scoring=c["scoring"], num_expert_group=c["num_expert_group"], topk_group=c["topk_group"],
               bias=c["bias"], routed_scaling_factor=c["routed_scaling_factor"])


@pytest.mark.parametrize("T,E,k,scoring,G,tg,bias_std,factor,renorm", [
    (1000, 256, 8, "sigmoid", 8, 4, 0.1, 2.5, True),     # DeepSeek-V3-shaped
    (333, 64, 6, "softmax", 8, 3, 0.0, 1.0, True),       # grouped, no bias
    (200, 160, 6, "softmax", 8, 3, 0.05, 16.0, True),
    (77, 1024, 8, "sigmoid", 0, 0, 0.2, 1.0, False),     # widest E, bias, no groups
    (64, 8, 2, "sigmoid", 0, 0, 0.0, 1.0, True),
    (50, 96, 4, "softmax", 32, 2, 0.3, 0.5, False),
    (1, 128, 8, "sigmoid", 64, 64, 0.1, 1.0, True),      # 64 groups of 2, all kept
])
def test_random(T, E, k, scoring, G, tg, bias_std, factor, renorm):
    logits = synthetic.random_logits(T, E, seed=T + E)
    bias = None
    if bias_std:
        bias = (bias_std * np.random.default_rng(E).standard_normal(E)).astype(np.float32)
    _check(logits, k, f"T={T} E={E} k={k} {scoring} G={G}/{tg} bias={bias_std} x{factor}", renormalize=renorm,
           scoring=scoring, num_expert_group=G, topk_group=tg, bias=bias, routed_scaling_factor=factor)


def test_ties_and_defaults():
    rng = np.random.default_rng(9)
    logits = rng.integers(-2, 3, size=(300, 32)).astype(np.float32)   # many equal logits
    bias = (rng.integers(-2, 3, size=32) * 0.125).astype(np.float32)
    _check(logits, 4, "integer logits, grouped", scoring="sigmoid", num_expert_group=8, topk_group=2, bias=bias)
    _check(logits, 4, "integer logits, softmax grouped", num_expert_group=4, topk_group=3)
    # the defaults take the softmax router's path and equal moe_route_topk
    logits = synthetic.random_logits(40, 16, seed=3)
    w, ids = _gpu(logits, 3)
    tw = torch.empty(40, 3, dtype=torch.float32, device=DEV)
    ti = torch.empty(40, 3, dtype=torch.int32, device=DEV)
    pkg.moe_route_topk(torch.from_numpy(logits).to(DEV), 3, True, tw, ti)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids, ti.cpu().numpy())
    np.testing.assert_array_equal(w, tw.cpu().numpy())


def test_bad_arguments_raise():
    logits = torch.zeros(4, 8, device=DEV)
    tw = torch.empty(4, 2, device=DEV)
    ti = torch.empty(4, 2, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        pkg.moe_route_select(logits, 2, tw, ti, num_expert_group=3, topk_group=1)
    with pytest.raises(ValueError):
        pkg.moe_route_select(logits, 2, tw, ti, num_expert_group=4, topk_group=5)
    with pytest.raises(ValueError):
        pkg.moe_route_select(logits, 2, tw, ti, scoring="tanh")
    with pytest.raises(ValueError):
        pkg.moe_route_select(logits, 2, tw, ti, routed_scaling_factor=float("inf"))
