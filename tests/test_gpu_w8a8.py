"""GPU W8A8 layer (per-channel int8 weights, per-token dynamic int8 activations; fused_moe
oracle/int8 page, select_int8_moe_backend) against the W8A8 oracle: activation codes and scales bit
for bit, the layer within the layer tolerance."""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import (DEV, act_f64, assert_layer_close, assert_w8a8_close, log, route_both, small_w8, to_dev_act,
                        workload_weights)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    pkg.lib()


# rows of up to 4096 values: one workgroup per row; 8192: a wave per row (no partial maxima)
@pytest.mark.parametrize("act,T,H", [("bf16", 37, 512), ("fp16", 5, 4096), ("bf16", 1000, 2048), ("bf16", 3, 8192)])
def test_activation_codes_bit_exact(act, T, H):
    xb = synthetic.random_activations(T, H, act, seed=T)
    xb[0] = 0                                              # a zero row: scale 0, codes 0
    x = to_dev_act(xb, act)
    q = torch.empty(T, H, dtype=torch.int8, device=DEV)
    s = torch.empty(T, dtype=torch.float32, device=DEV)
    pkg.moe_quantize_act_int8(x, q, s)
    torch.cuda.synchronize()
    qr, sr = oracle.quantize_act_int8_rows(act_f64(xb, act))
    np.testing.assert_array_equal(q.cpu().numpy(), qr)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), sr.view(np.uint32))


def _run(W, xb, act, logits, k, bm=0, S=0, woi=False):
    T = xb.shape[0]
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    x = to_dev_act(xb, act)
    out = torch.empty_like(x)
    E = W.E - S
    ws = torch.empty(pkg.moe_w8a8_workspace_bytes(T, W.H, W.I, E, k, bm, S, woi), dtype=torch.uint8, device=DEV)
    pkg.moe_w8a8_forward(x, W.w13, W.s13, W.w2, W.s2, tw, ti, out, ws, num_shared_experts=S,
                         apply_router_weight_on_input=woi, block_m=bm)
    torch.cuda.synchronize()
    x64 = act_f64(xb, act)
    ref = oracle.moe_forward_w8a8(x64, W.q13, W.hs13, W.q2, W.hs2, w_ref, ids_ref, weight_on_input=woi, num_shared=S)
    got = out.float().cpu().numpy().astype(np.float64)
    check = lambda what: assert_w8a8_close(got, ref, x64, W, w_ref, ids_ref, what, woi, S)  # noqa: E731
    return got, ref, check


@pytest.mark.parametrize("act,T,bm,pad", [("bf16", 5, 0, True), ("fp16", 61, 32, False), ("bf16", 130, 64, True),
                                          ("bf16", 700, 256, True), ("fp16", 300, 128, False), ("bf16", 1, 16, True)])
def test_layer_small(act, T, bm, pad):
    E, k, H, I = 8, 2, 512, 1024
    log(f"[w8a8] act={act} T={T} block_m={bm}")
    W = small_w8(E, H, I, seed=13, pad=pad)
    xb = synthetic.random_activations(T, H, act, seed=T)
    logits = synthetic.random_logits(T, E, seed=T + 1)
    got, ref, check = _run(W, xb, act, logits, k, bm)
    check(f"w8a8 {act} T={T} bm={bm}")


@pytest.mark.parametrize("T,bm", [(3, 16), (40, 32)])
def test_layer_odd_shapes(T, bm):
    """The 16/32-row streaming GEMMs with H = 3 x 128 (three column tiles) and I = 5 x 128 (K parts of
    uneven length)."""
    E, k, H, I = 8, 2, 384, 640
    log(f"[w8a8] odd shapes T={T} block_m={bm}")
    W = small_w8(E, H, I, seed=17, pad=True)
    xb = synthetic.random_activations(T, H, "bf16", seed=T + 7)
    logits = synthetic.random_logits(T, E, seed=T + 8)
    got, ref, check = _run(W, xb, "bf16", logits, k, bm)
    check(f"w8a8 odd shapes T={T} bm={bm}")


def test_layer_options():
    E, k, H, I, T, S = 8, 3, 256, 384, 40, 1
    W = small_w8(E + S, H, I, seed=17, pad=True)
    xb = synthetic.random_activations(T, H, "bf16", seed=18)
    logits = synthetic.random_logits(T, E, seed=19)
    for woi in (False, True):
        got, ref, check = _run(W, xb, "bf16", logits, k, S=S, woi=woi)
        check(f"w8a8 shared={S} woi={woi}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [8, 64])
def test_mixtral_decode_w8a8(T):
    wl = synthetic.WORKLOADS["mixtral_decode"]
    W = workload_weights(wl)
    xb = synthetic.activations(wl, T)
    logits = synthetic.router_logits(wl, T)
    got, ref, check = _run(W, xb, wl.act, logits, wl.k)
    check(f"w8a8 mixtral decode T={T}")
    again, _, _ = _run(W, xb, wl.act, logits, wl.k)
    assert np.array_equal(got, again), "two runs differ bitwise"
    # the allowance is for a few code steps: almost every element meets the plain layer tolerance
    base = 2e-2 * np.abs(ref) + 1e-3
    assert (np.abs(got - ref) > base).mean() < 1e-3


def test_apply_equals_route_then_forward():
    E, k, H, I, T = 16, 4, 256, 256, 33
    W = small_w8(E, H, I, seed=21)
    xb = synthetic.random_activations(T, H, "bf16", seed=22)
    logits = synthetic.random_logits(T, E, seed=23)
    got, _, _ = _run(W, xb, "bf16", logits, k)
    x = to_dev_act(xb, "bf16")
    out = torch.empty_like(x)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(pkg.moe_w8a8_workspace_bytes(T, H, I, E, k), dtype=torch.uint8, device=DEV)
    pkg.moe_w8a8_apply(x, torch.from_numpy(logits).to(DEV), W.w13, W.s13, W.w2, W.s2, tw, ti, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), got)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [1024, 4096])
def test_mixtral_prefill_w8a8_sampled(T):
    """Mixtral prefill (uneven expert loads, 256-row blocks, the big int8 GEMMs): every output row depends
    only on its own token, so the oracle checks a sample of 8 rows spread over the batch."""
    wl = synthetic.WORKLOADS["mixtral_prefill"]
    W = workload_weights(wl)
    xb = synthetic.activations(wl, T)
    logits = synthetic.router_logits(wl, T)
    k = wl.k
    assert pkg.moe_w8a16_block_m(T, wl.H, wl.I, wl.E, k) == 256
    log(f"[w8a8] mixtral prefill T={T}")
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    x = to_dev_act(xb, wl.act)
    out = torch.empty_like(x)
    ws = torch.empty(pkg.moe_w8a8_workspace_bytes(T, W.H, W.I, W.E, k), dtype=torch.uint8, device=DEV)
    pkg.moe_w8a8_forward(x, W.w13, W.s13, W.w2, W.s2, tw, ti, out, ws)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, T - 1, 8).astype(int))
    x64 = act_f64(xb[rows], wl.act)
    ref = oracle.moe_forward_w8a8(x64, W.q13, W.hs13, W.q2, W.hs2, w_ref[rows], ids_ref[rows])
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    assert_w8a8_close(got, ref, x64, W, w_ref[rows], ids_ref[rows], f"w8a8 mixtral prefill T={T} sampled rows")
