"""moe_w8a16_forward_noalloc (the forward on the library's static device workspace, for callers
that cannot allocate) against moe_w8a16_forward with a caller workspace: the same bytes, on
consecutive calls whose second one is smaller, plus the oracle's tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import binding as B
from weight_quantized_mixture_amd import synthetic

from moe_cases import DEV, assert_layer_close, log, ref_w8, route_both, small_w8, to_dev_act

pytestmark = pytest.mark.gpu


def _both(W, xb, act, logits, k, bm):
    T = xb.shape[0]
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    x = to_dev_act(xb, act)
    out_ws = torch.empty_like(x)
    ws = torch.empty(max(pkg.moe_w8a16_workspace_bytes(T, W.H, W.I, W.E, k, bm), 256), dtype=torch.uint8,
                     device=DEV)
    pkg.moe_w8a16_forward(x, W.w13, W.s13, W.w2, W.s2, tw, ti, out_ws, ws, bm)
    out_na = torch.full_like(x, float("nan"))
    B.moe_w8a16_forward_noalloc(x, W.w13, W.s13, W.w2, W.s2, tw, ti, out_na, bm)
    torch.cuda.synchronize()
    return (out_ws.float().cpu().numpy().astype(np.float64), out_na.float().cpu().numpy().astype(np.float64),
            w_ref, ids_ref)


@pytest.mark.parametrize("E,k,H,I,T1,bm1,T2,bm2", [(8, 2, 512, 1024, 61, 32, 9, 16),
                                                  (16, 4, 384, 640, 130, 64, 3, 0),
                                                  (8, 2, 256, 512, 300, 256, 40, 0)])
def test_noalloc_matches_forward_twice(E, k, H, I, T1, bm1, T2, bm2):
    assert torch.cuda.is_available()
    W = small_w8(E, H, I, seed=E + H, pad=True)
    for T, bm in ((T1, bm1), (T2, bm2)):
        log(f"[noalloc] E={E} k={k} H={H} I={I} T={T} block_m={bm}")
        xb = synthetic.random_activations(T, H, "bf16", seed=T + 7)
        logits = synthetic.random_logits(T, E, seed=T + 8)
        got_ws, got_na, w_ref, ids_ref = _both(W, xb, "bf16", logits, k, bm)
        assert np.array_equal(got_ws, got_na), f"no-alloc forward differs from the workspace forward at T={T}"
        assert_layer_close(got_na, ref_w8(W, xb, "bf16", w_ref, ids_ref), f"no-alloc T={T} bm={bm}")


def test_noalloc_rejects_batches_beyond_the_scratch():
    """A batch whose workspace exceeds the static array fails before anything is launched."""
    E, k, H, I, T = 8, 2, 4096, 14336, 1024
    assert pkg.moe_w8a16_workspace_bytes(T, H, I, E, k, 0) > B.MOE_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(0x100000)
    r = pkg.lib().moe_w8a16_forward_noalloc(p, 0, T, H, I, E, k, p, p, 0, p, p, 0, p, p, 0, p, None)
    assert r == B.MOE_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in pkg.lib().moe_last_error()
