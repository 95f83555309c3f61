"""GPU parity of the group-wise W4A16 layer against the fp64 oracle (same
layer tolerance as W8A16; packed codes, fp16 scales and zeros bit for bit)."""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import DEV, W4Weights, act_f64, assert_layer_close, log, route_both, to_dev_act, workload_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    pkg.lib()


def _run(W, xb, act, logits, k, block_m=0):
    T = xb.shape[0]
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    np.testing.assert_array_equal(ti.cpu().numpy(), ids_ref)
    x = to_dev_act(xb, act)
    out = torch.empty_like(x)
    ws = torch.empty(max(pkg.moe_w4a16_workspace_bytes(T, W.H, W.I, W.E, k, block_m), 256),
                     dtype=torch.uint8, device=DEV)
    pkg.moe_w4a16_forward(x, W.qw13, W.sc13, W.qz13, W.qw2, W.sc2, W.qz2, W.g, tw, ti, out, ws, block_m)
    torch.cuda.synchronize()
    ref = oracle.moe_forward_w4(act_f64(xb, act), W.h["qw13"], W.h["sc13"], W.h["qz13"], W.h["qw2"],
                                W.h["sc2"], W.h["qz2"], W.g, w_ref, ids_ref)
    return out.float().cpu().numpy().astype(np.float64), ref


@pytest.mark.parametrize("act,bm,T", [("fp16", 0, 21), ("bf16", 0, 21), ("fp16", 64, 90), ("fp16", 16, 3)])
def test_w4_small(act, bm, T):
    E, k, H, I, g = 8, 3, 256, 384, 128
    log(f"[w4] act={act} bm={bm} T={T}")
    fn = lambda which, e: synthetic.random_master((2 * I, H) if which == "w13" else (H, I),  # noqa: E731
                                                  100 + e, tag=70 if which == "w13" else 71)
    W = W4Weights(E, H, I, g, fn)
    assert W.mismatch == 0
    xb = synthetic.random_activations(T, H, act, seed=T)
    logits = synthetic.random_logits(T, E, seed=T + 2)
    got, ref = _run(W, xb, act, logits, k, bm)
    assert_layer_close(got, ref, f"w4 small {act} bm={bm} T={T}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [8, 256])
def test_w4a16_workload(T):
    wl = synthetic.WORKLOADS["w4a16"]
    W = workload_weights(wl)
    assert W.mismatch == 0, "GPU uint4 codes / scales / zeros differ from the oracle"
    xb = synthetic.activations(wl, T)
    logits = synthetic.router_logits(wl, T)
    got, ref = _run(W, xb, wl.act, logits, wl.k)
    assert_layer_close(got, ref, f"w4a16 T={T}")


def test_w4_apply_from_logits():
    E, k, H, I, g, T = 8, 3, 256, 384, 128, 33
    fn = lambda which, e: synthetic.random_master((2 * I, H) if which == "w13" else (H, I),  # noqa: E731
                                                  200 + e, tag=72 if which == "w13" else 73)
    W = W4Weights(E, H, I, g, fn)
    xb = synthetic.random_activations(T, H, "fp16", seed=5)
    logits = synthetic.random_logits(T, E, seed=6)
    got, ref = _run(W, xb, "fp16", logits, k)
    x = to_dev_act(xb, "fp16")
    out = torch.empty_like(x)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(pkg.moe_w4a16_workspace_bytes(T, H, I, E, k, 0), dtype=torch.uint8, device=DEV)
    pkg.moe_w4a16_apply(x, torch.from_numpy(logits).to(DEV), True, W.qw13, W.sc13, W.qz13, W.qw2, W.sc2, W.qz2, g,
                        tw, ti, out, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), got)
    assert_layer_close(got, ref, "w4 apply from logits")


@pytest.mark.parametrize("act,bm,T,H,I,g", [("fp16", 32, 45, 256, 384, 128), ("bf16", 32, 45, 256, 384, 128),
                                            ("bf16", 16, 7, 384, 256, 128), ("fp16", 16, 30, 384, 384, 128),
                                            ("fp16", 32, 61, 512, 512, 256), ("bf16", 16, 1, 512, 512, 256),
                                            ("fp16", 16, 5, 2560, 256, 128), ("bf16", 32, 40, 4096, 256, 128),
                                            ("fp16", 16, 3, 4224, 256, 128)])
def test_w4_blocks_of_16_and_32(act, bm, T, H, I, g):
    # GEMM1 of 16/32-row blocks copies each wave's scales and zero words of
    # the whole K into LDS once and streams the packed rows through the ring:
    # odd group counts per row (H / g = 3) put the scale spans at odd element
    # offsets, g = 256 spans two K steps, 20 and 32 groups per row take the
    # larger scale area, and 33 groups the streaming kernel instead
    E, k = 8, 3
    log(f"[w4 dma] act={act} bm={bm} T={T} H={H} I={I} g={g}")
    fn = lambda which, e: synthetic.random_master((2 * I, H) if which == "w13" else (H, I),  # noqa: E731
                                                  300 + e, tag=74 if which == "w13" else 75)
    W = W4Weights(E, H, I, g, fn)
    assert W.mismatch == 0
    xb = synthetic.random_activations(T, H, act, seed=T + 11)
    logits = synthetic.random_logits(T, E, seed=T + 12)
    got, ref = _run(W, xb, act, logits, k, bm)
    assert_layer_close(got, ref, f"w4 dma {act} bm={bm} T={T} H={H} I={I} g={g}")
