"""GPU parity of the whole layer (route + align + GEMM1/SiLU + GEMM2 + combine)
against the fp64 oracle, to the layer tolerance
max|gpu - ref| <= 2e-2 max|ref| and |gpu - ref| <= 2e-2 |ref| + 1e-3 per element,
with router ids bit for bit.  Full-size workloads use every token when the
oracle is quick and an even sample of tokens for the long prefill."""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import (DEV, act_f64, assert_layer_close, log, ref_w8, route_both, run_w8_layer, small_w8,
                       to_dev_act, workload_weights)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    pkg.lib()


def _check_routing(ti, tw, ids_ref, w_ref):
    np.testing.assert_array_equal(ti, ids_ref)
    np.testing.assert_allclose(tw, w_ref, rtol=0, atol=1e-6)


def test_tiny_workload():
    wl = synthetic.WORKLOADS["tiny"]
    W = workload_weights(wl)
    assert W.mismatch == 0
    T = wl.tokens[0]
    xb = synthetic.activations(wl, T)
    logits = synthetic.router_logits(wl, T)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, wl.act, logits, wl.k)
    _check_routing(ti, tw, ids_ref, w_ref)
    assert_layer_close(got, ref_w8(W, xb, wl.act, w_ref, ids_ref), "tiny T=16")


@pytest.mark.parametrize("act,bm,T,pad", [("bf16", 0, 37, False), ("fp16", 0, 37, True), ("bf16", 16, 5, True),
                                          ("bf16", 32, 61, False), ("bf16", 32, 61, True), ("bf16", 64, 130, True),
                                          ("fp16", 48, 77, False), ("bf16", 128, 300, True), ("fp16", 64, 200, False),
                                          ("bf16", 256, 700, True), ("fp16", 256, 333, False), ("bf16", 256, 9, True)])
def test_ragged_shapes(act, bm, T, pad):
    E, k, H, I = 8, 2, 512, 1024
    log(f"[layer] ragged act={act} bm={bm} T={T} padded_rows={pad}")
    W = small_w8(E, H, I, seed=7, pad=pad)
    assert W.mismatch == 0
    xb = synthetic.random_activations(T, H, act, seed=T)
    logits = synthetic.random_logits(T, E, seed=T + 1)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, act, logits, k, block_m=bm)
    _check_routing(ti, tw, ids_ref, w_ref)
    assert_layer_close(got, ref_w8(W, xb, act, w_ref, ids_ref), f"ragged {act} bm={bm} T={T} pad={pad}")


@pytest.mark.parametrize("H,I,T,bm", [(384, 256, 1, 0), (896, 256, 1, 0), (384, 512, 20, 32), (4224, 256, 130, 64),
                                      (640, 384, 3, 16)])
def test_hidden_not_multiple_of_256(H, I, T, bm):
    """H a multiple of 128 but not of 256 on the integer GEMM2 of 16-64-row blocks: every column of
    y is written (the kernel takes 128 columns per workgroup there, not 256)."""
    E, k = 8, 2
    log(f"[layer] H={H} I={I} T={T} block_m={bm}")
    W = small_w8(E, H, I, seed=H + T, pad=True)
    xb = synthetic.random_activations(T, H, "bf16", seed=H)
    logits = synthetic.random_logits(T, E, seed=H + 1)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, "bf16", logits, k, block_m=bm)
    _check_routing(ti, tw, ids_ref, w_ref)
    assert_layer_close(got, ref_w8(W, xb, "bf16", w_ref, ids_ref), f"H={H} T={T} bm={bm}")


def test_block256_odd_hidden():
    """256-row blocks with H not a multiple of 256 (the GEMM2 tile): the generic tiled kernel."""
    E, k, H, I, T = 4, 2, 384, 256, 200
    log(f"[layer] block_m=256 H={H} I={I} T={T}")
    W = small_w8(E, H, I, seed=23, pad=True)
    xb = synthetic.random_activations(T, H, "bf16", seed=24)
    logits = synthetic.random_logits(T, E, seed=25)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, "bf16", logits, k, block_m=256)
    assert_layer_close(got, ref_w8(W, xb, "bf16", w_ref, ids_ref), "block_m=256 H=384")


def test_edge_cases_routing_shapes():
    H, I = 256, 256
    # k = E, one token, renormalize off
    W = small_w8(4, H, I, seed=11)
    xb = synthetic.random_activations(1, H, "bf16", seed=12)
    logits = synthetic.random_logits(1, 4, seed=13)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, "bf16", logits, 4, renormalize=False)
    _check_routing(ti, tw, ids_ref, w_ref)
    assert_layer_close(got, ref_w8(W, xb, "bf16", w_ref, ids_ref), "k=E T=1")
    # every token to one expert (others empty)
    W = small_w8(16, H, I, seed=14)
    xb = synthetic.random_activations(50, H, "bf16", seed=15)
    bias = np.zeros(16, np.float32); bias[9] = 30.0
    logits = synthetic.random_logits(50, 16, seed=16, bias=bias)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, "bf16", logits, 1)
    assert np.all(ti == 9)
    assert_layer_close(got, ref_w8(W, xb, "bf16", w_ref, ids_ref), "all tokens to one expert")
    # many experts, few tokens (most experts empty)
    W = small_w8(64, H, I, seed=17)
    xb = synthetic.random_activations(2, H, "bf16", seed=18)
    logits = synthetic.random_logits(2, 64, seed=19)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, "bf16", logits, 6)
    assert_layer_close(got, ref_w8(W, xb, "bf16", w_ref, ids_ref), "E=64 T=2")


def test_inplace_and_determinism():
    E, k, H, I, T = 8, 2, 256, 384, 40
    W = small_w8(E, H, I, seed=21)
    xb = synthetic.random_activations(T, H, "bf16", seed=22)
    logits = synthetic.random_logits(T, E, seed=23)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, "bf16", logits, k, inplace=True)
    assert_layer_close(got, ref_w8(W, xb, "bf16", w_ref, ids_ref), "inplace out == x")
    outs = []
    for _ in range(2):
        g2, *_ = run_w8_layer(W, xb, "bf16", logits, k)
        outs.append(g2)
    assert np.array_equal(outs[0], outs[1]), "two runs differ bitwise"
    assert np.array_equal(outs[0], got), "inplace result differs from out-of-place"


def test_out_of_range_ids_dropped():
    E, k, H, I, T = 8, 2, 256, 256, 6
    W = small_w8(E, H, I, seed=31)
    xb = synthetic.random_activations(T, H, "bf16", seed=32)
    ids = np.array([[0, 9], [-1, 3], [2, 2], [7, 8], [1, 0], [5, 4]], np.int32)
    w = np.full((T, k), 0.5, np.float32)
    x = to_dev_act(xb, "bf16")
    out = torch.empty_like(x)
    ws = torch.empty(pkg.moe_w8a16_workspace_bytes(T, H, I, E, k, 0), dtype=torch.uint8, device=DEV)
    pkg.moe_w8a16_forward(x, W.w13, W.s13, W.w2, W.s2, torch.from_numpy(w).to(DEV),
                          torch.from_numpy(ids).to(DEV), out, ws)
    torch.cuda.synchronize()
    ref = oracle.moe_forward_w8(act_f64(xb, "bf16"), W.q13, W.hs13, W.q2, W.hs2, w.astype(np.float64), ids)
    assert_layer_close(out.float().cpu().numpy().astype(np.float64), ref, "out-of-range ids")


def test_zero_tokens():
    H, I, E, k = 256, 256, 8, 2
    W = small_w8(E, H, I, seed=41)
    x = torch.empty(0, H, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    tw = torch.empty(0, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(0, k, dtype=torch.int32, device=DEV)
    pkg.moe_w8a16_forward(x, W.w13, W.s13, W.w2, W.s2, tw, ti, torch.empty_like(x), ws)
    torch.cuda.synchronize()


def test_bad_shapes_raise():
    W = small_w8(2, 256, 256, seed=1)
    x = torch.zeros(4, 256, dtype=torch.bfloat16, device=DEV)
    tw = torch.zeros(4, 2, dtype=torch.float32, device=DEV)
    ti = torch.zeros(4, 2, dtype=torch.int32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        pkg.moe_w8a16_forward(x, W.w13, W.s13, W.w2, W.s2, tw, ti, torch.empty_like(x), ws)   # workspace


# ---- full-size workloads ------------------------------------------------------


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,bm", [(1, 0), (8, 0), (32, 0), (64, 0), (64, 64), (256, 0)])
def test_mixtral_decode(T, bm):
    """Every token against the oracle; a second run must give the same bytes (the integer GEMM2 of
    16/32/64/128-row blocks with its split-K partials summed in a fixed order; T = 256 takes 128-row
    blocks, GEMM2 on their 64-row halves)."""
    wl = synthetic.WORKLOADS["mixtral_decode"]
    W = workload_weights(wl)
    assert W.mismatch == 0, "GPU int8 codes or scales differ from the oracle"
    xb = synthetic.activations(wl, T)
    logits = synthetic.router_logits(wl, T)
    log(f"[layer] mixtral decode T={T} block_m={bm or pkg.moe_w8a16_block_m(T, wl.H, wl.I, wl.E, wl.k)} "
        f"splits={pkg.moe_w8a16_splits(T, wl.H, wl.I, wl.E, wl.k, bm)}")
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, wl.act, logits, wl.k, block_m=bm)
    _check_routing(ti, tw, ids_ref, w_ref)
    again, *_ = run_w8_layer(W, xb, wl.act, logits, wl.k, block_m=bm)
    assert np.array_equal(got, again), "two runs differ bitwise"
    assert_layer_close(got, ref_w8(W, xb, wl.act, w_ref, ids_ref), f"mixtral decode T={T} bm={bm}")


def _edge_block_tokens(ids, E, k, block_m):
    """Tokens routed through the first or the last align block of every expert."""
    sorted_ids, block_expert, npad = oracle.align_block(ids, E, block_m)
    tk = ids.size
    toks = []
    for e in range(E):
        blocks = np.nonzero(block_expert[:npad // block_m] == e)[0]
        for b in {int(blocks[0]), int(blocks[-1])} if blocks.size else ():
            f = sorted_ids[b * block_m:(b + 1) * block_m]
            toks.append(f[f < tk] // k)
    return np.unique(np.concatenate(toks))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,nsample", [(1024, 96), (4096, 64)])
def test_mixtral_prefill_sampled(T, nsample):
    """256-row tiles: every token of the first and the last 256-row block of each expert (all row
    positions of a full tile and of the ragged last tile), plus an even sample; a second run gives
    the same bytes (GEMM2 split into 2 K parts at T=1024, one at T=4096)."""
    wl = synthetic.WORKLOADS["mixtral_prefill"]
    W = workload_weights(wl)
    assert W.mismatch == 0
    xb = synthetic.activations(wl, T)
    logits = synthetic.router_logits(wl, T)
    bm = pkg.moe_w8a16_block_m(T, wl.H, wl.I, wl.E, wl.k)
    log(f"[layer] mixtral prefill T={T} block_m={bm} splits={pkg.moe_w8a16_splits(T, wl.H, wl.I, wl.E, wl.k, 0)}")
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, wl.act, logits, wl.k)
    _check_routing(ti, tw, ids_ref, w_ref)
    again, *_ = run_w8_layer(W, xb, wl.act, logits, wl.k)
    assert np.array_equal(got, again), "two runs differ bitwise"
    edge = _edge_block_tokens(ids_ref, wl.E, wl.k, bm)
    rows = np.unique(np.concatenate([[0, T - 1], np.linspace(0, T - 1, nsample).astype(int), edge]))
    log(f"[layer] checking {rows.size} tokens ({edge.size} from the edge blocks)")
    assert_layer_close(got[rows], ref_w8(W, xb, wl.act, w_ref, ids_ref, rows=rows),
                       f"mixtral prefill T={T} ({rows.size} tokens)")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [16, 512])
def test_fine_grained(T):
    wl = synthetic.WORKLOADS["fine_grained"]
    W = workload_weights(wl)
    assert W.mismatch == 0
    xb = synthetic.activations(wl, T)
    logits = synthetic.router_logits(wl, T)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, wl.act, logits, wl.k)
    _check_routing(ti, tw, ids_ref, w_ref)
    assert_layer_close(got, ref_w8(W, xb, wl.act, w_ref, ids_ref), f"fine-grained T={T}")


# fused routing + align up to 8 tokens (8 x 1024 on the arg-max router at the limit), separate launches
# past it (9 x 1024, 16 x 64, 64 x 128, 65 tokens, 300 and 600 tokens)
@pytest.mark.parametrize("T,E,k,act", [(1, 8, 2, "bf16"), (8, 64, 6, "fp16"), (37, 8, 2, "fp16"),
                                       (300, 16, 4, "bf16"), (600, 8, 2, "bf16"), (5, 128, 8, "fp16"),
                                       (20, 96, 4, "bf16"), (64, 8, 2, "bf16"), (16, 64, 6, "bf16"),
                                       (64, 128, 8, "fp16"), (8, 1024, 4, "bf16"), (65, 8, 2, "bf16"),
                                       (9, 1024, 2, "bf16")])
def test_apply_from_logits_matches_route_then_forward(T, E, k, act):
    """moe_w8a16_apply (routing fused with align up to 8 tokens) equals route + forward bit for bit."""
    H, I = (256, 384) if E <= 128 else (128, 128)
    W = small_w8(E, H, I, seed=51, pad=True)
    xb = synthetic.random_activations(T, H, act, seed=52)
    logits = synthetic.random_logits(T, E, seed=53)
    got, tw, ti, w_ref, ids_ref = run_w8_layer(W, xb, act, logits, k)
    x = to_dev_act(xb, act)
    dl = torch.from_numpy(logits).to(DEV)
    out = torch.empty_like(x)
    tw2 = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti2 = torch.empty(T, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(pkg.moe_w8a16_workspace_bytes(T, H, I, E, k, 0), dtype=torch.uint8, device=DEV)
    pkg.moe_w8a16_apply(x, dl, True, W.w13, W.s13, W.w2, W.s2, tw2, ti2, out, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ti2.cpu().numpy(), ti)
    np.testing.assert_array_equal(tw2.cpu().numpy(), tw)
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), got)
    assert_layer_close(got, ref_w8(W, xb, act, w_ref, ids_ref), f"apply T={T} E={E} k={k}")
