"""GPU parity of the layer with the select_experts / fused_experts options against the oracle:
grouped and biased routing from logits (ids bit for bit), shared experts, and the routing weight
applied to the input, for the int8 and the uint4 weights, at several align block sizes."""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import DEV, W4Weights, act_f64, assert_layer_close, log, small_w8, to_dev_act

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    pkg.lib()


def _route_opts(case, E, seed):
    scoring, G, tg, bias_std, factor = case
    bias = None
    if bias_std:
        bias = (bias_std * np.random.default_rng(seed).standard_normal(E)).astype(np.float32)
    return dict(renormalize=True, scoring=scoring, num_expert_group=G, topk_group=tg, bias=bias,
                routed_scaling_factor=factor)


def _apply_w8(W, xb, act, logits, k, S, woi, ro, bm):
    T = xb.shape[0]
    x = to_dev_act(xb, act)
    out = torch.empty_like(x)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    E = W.E - S
    ws = torch.empty(pkg.moe_w8a16_workspace_bytes_ex(T, W.H, W.I, E, k, bm, S, woi), dtype=torch.uint8,
                     device=DEV)
    b = None if ro["bias"] is None else torch.from_numpy(ro["bias"]).to(DEV)
    pkg.moe_w8a16_apply_ex(x, torch.from_numpy(logits).to(DEV), W.w13, W.s13, W.w2, W.s2, tw, ti, out, ws,
                           renormalize=ro["renormalize"], scoring=ro["scoring"], num_expert_group=ro["num_expert_group"],
                           topk_group=ro["topk_group"], e_score_correction_bias=b,
                           routed_scaling_factor=ro["routed_scaling_factor"], num_shared_experts=S,
                           apply_router_weight_on_input=woi, block_m=bm)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), tw.cpu().numpy(), ti.cpu().numpy()


ROUTES = {"deepseek": ("sigmoid", 4, 2, 0.1, 2.5), "grouped_softmax": ("softmax", 4, 3, 0.0, 1.0),
          "plain": ("softmax", 0, 0, 0.0, 1.0)}


@pytest.mark.parametrize("route,S,woi,T,bm,act", [
    ("deepseek", 1, False, 40, 0, "bf16"), ("deepseek", 2, False, 300, 0, "bf16"),
    ("grouped_softmax", 0, True, 33, 16, "bf16"), ("plain", 1, True, 61, 32, "fp16"),
    ("deepseek", 1, True, 130, 64, "bf16"), ("plain", 2, False, 700, 256, "bf16"),
    ("grouped_softmax", 1, True, 5, 0, "bf16"), ("plain", 0, True, 3, 0, "fp16")])
def test_w8_apply_ex(route, S, woi, T, bm, act):
    E, k, H, I = 16, 4, 512, 512
    log(f"[options] w8 route={route} shared={S} weight_on_input={woi} T={T} block_m={bm} {act}")
    W = small_w8(E + S, H, I, seed=S * 10 + T, pad=True)
    assert W.mismatch == 0
    xb = synthetic.random_activations(T, H, act, seed=T)
    logits = synthetic.random_logits(T, E, seed=T + 1)
    ro = _route_opts(ROUTES[route], E, T)
    got, tw, ti = _apply_w8(W, xb, act, logits, k, S, woi, ro, bm)
    w_ref, ids_ref = oracle.route_select(logits, k, **ro)
    np.testing.assert_array_equal(ti, ids_ref)
    np.testing.assert_allclose(tw, w_ref, rtol=0, atol=1e-6 * ro["routed_scaling_factor"])
    ref = oracle.moe_forward_w8(act_f64(xb, act), W.q13, W.hs13, W.q2, W.hs2, w_ref, ids_ref,
                                weight_on_input=woi, num_shared=S)
    assert_layer_close(got, ref, f"w8 options {route} S={S} woi={woi} T={T} bm={bm}")


def test_w8_ex_defaults_equal_plain_calls():
    """With no options the _ex calls give the plain calls' bytes."""
    E, k, H, I, T = 8, 2, 256, 384, 37
    W = small_w8(E, H, I, seed=77, pad=True)
    xb = synthetic.random_activations(T, H, "bf16", seed=78)
    logits = synthetic.random_logits(T, E, seed=79)
    got_ex, tw_ex, ti_ex = _apply_w8(W, xb, "bf16", logits, k, 0, False, _route_opts(ROUTES["plain"], E, 0), 0)
    x = to_dev_act(xb, "bf16")
    out = torch.empty_like(x)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(pkg.moe_w8a16_workspace_bytes(T, H, I, E, k, 0), dtype=torch.uint8, device=DEV)
    pkg.moe_w8a16_apply(x, torch.from_numpy(logits).to(DEV), True, W.w13, W.s13, W.w2, W.s2, tw, ti, out, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ti.cpu().numpy(), ti_ex)
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), got_ex)
    # forward_ex with the routing the apply produced, shared experts off, weight on the input off
    out2 = torch.empty_like(x)
    pkg.moe_w8a16_forward_ex(x, W.w13, W.s13, W.w2, W.s2, tw, ti, out2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)


@pytest.mark.parametrize("S,woi,T,bm", [(1, False, 21, 0), (1, True, 90, 64), (0, True, 3, 16)])
def test_w4_forward_ex(S, woi, T, bm):
    E, k, H, I, g = 8, 3, 256, 384, 128
    log(f"[options] w4 shared={S} weight_on_input={woi} T={T} block_m={bm}")
    fn = lambda which, e: synthetic.random_master((2 * I, H) if which == "w13" else (H, I), 900 + e,  # noqa: E731
                                                  tag=70 if which == "w13" else 71)
    W = W4Weights(E + S, H, I, g, fn)
    assert W.mismatch == 0
    xb = synthetic.random_activations(T, H, "fp16", seed=T)
    logits = synthetic.random_logits(T, E, seed=T + 2)
    w_ref, ids_ref = oracle.route_softmax_topk(logits, k, True)
    x = to_dev_act(xb, "fp16")
    out = torch.empty_like(x)
    tw = torch.from_numpy(w_ref.astype(np.float32)).to(DEV)
    ti = torch.from_numpy(ids_ref).to(DEV)
    ws = torch.empty(pkg.moe_w4a16_workspace_bytes_ex(T, H, I, E, k, bm, S, woi), dtype=torch.uint8, device=DEV)
    pkg.moe_w4a16_forward_ex(x, W.qw13, W.sc13, W.qz13, W.qw2, W.sc2, W.qz2, g, tw, ti, out, ws,
                             num_shared_experts=S, apply_router_weight_on_input=woi, block_m=bm)
    torch.cuda.synchronize()
    ref = oracle.moe_forward_w4(act_f64(xb, "fp16"), W.h["qw13"], W.h["sc13"], W.h["qz13"], W.h["qw2"], W.h["sc2"],
                                W.h["qz2"], g, w_ref.astype(np.float32).astype(np.float64), ids_ref,
                                weight_on_input=woi, num_shared=S)
    assert_layer_close(out.float().cpu().numpy().astype(np.float64), ref, f"w4 options S={S} woi={woi} T={T}")


def test_options_argument_errors():
    W = small_w8(4, 256, 256, seed=5)
    x = torch.zeros(4, 256, dtype=torch.bfloat16, device=DEV)
    tw = torch.zeros(4, 2, device=DEV)
    ti = torch.zeros(4, 2, dtype=torch.int32, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        pkg.moe_w8a16_forward_ex(x, W.w13, W.s13, W.w2, W.s2, tw, ti, torch.empty_like(x), ws, num_shared_experts=4)
    with pytest.raises(ValueError):       # logits must cover the routed experts only
        pkg.moe_w8a16_apply_ex(x, torch.zeros(4, 4, device=DEV), W.w13, W.s13, W.w2, W.s2, tw, ti,
                               torch.empty_like(x), ws, num_shared_experts=1)
