"""Shared builders for the GPU parity tests: seeded inputs on the host (the
same bytes go to the GPU and to the oracle), quantization on both sides, and
a per-session cache of the large weight sets."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic
from weight_quantized_mixture_amd.layer import padded_rows

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None


def log(msg):
    print(msg, flush=True)


def to_dev_act(bits: np.ndarray, act: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if act == "bf16" else torch.float16)
    return t.to(DEV)


def act_f64(bits, act):
    return oracle.act_bits_to_f64(bits, act)


class W8Weights:
    """int8 expert weights quantized on the GPU (K1) and by the oracle, compared bit for bit."""

    def __init__(self, E, H, I, master_fn, pad=False):
        self.E, self.H, self.I = E, H, I
        self.w13 = torch.empty(E, 2 * I, H, dtype=torch.int8, device=DEV)
        self.s13 = torch.empty(E, 2 * I, dtype=torch.float32, device=DEV)
        self.w2 = torch.empty(E, H, I, dtype=torch.int8, device=DEV)
        self.pad = pad
        self.s2 = torch.empty(E, H, dtype=torch.float32, device=DEV)
        self.q13 = np.empty((E, 2 * I, H), np.int8)
        self.hs13 = np.empty((E, 2 * I), np.float32)
        self.q2 = np.empty((E, H, I), np.int8)
        self.hs2 = np.empty((E, H), np.float32)
        self.mismatch = 0
        for e in range(E):
            m13 = master_fn("w13", e)
            m2 = master_fn("w2", e)
            d13 = torch.from_numpy(m13).to(DEV)
            d2 = torch.from_numpy(m2).to(DEV)
            pkg.moe_quantize_weights_int8(d13.view(1, 2 * I, H), self.w13[e:e + 1], self.s13[e:e + 1])
            pkg.moe_quantize_weights_int8(d2.view(1, H, I), self.w2[e:e + 1], self.s2[e:e + 1])
            self.q13[e], self.hs13[e] = oracle.quantize_int8_rows(m13)
            self.q2[e], self.hs2[e] = oracle.quantize_int8_rows(m2)
            torch.cuda.synchronize()
            del d13, d2
            if not (np.array_equal(self.w13[e].cpu().numpy(), self.q13[e])
                    and np.array_equal(self.s13[e].cpu().numpy().view(np.uint32), self.hs13[e].view(np.uint32))
                    and np.array_equal(self.w2[e].cpu().numpy(), self.q2[e])
                    and np.array_equal(self.s2[e].cpu().numpy().view(np.uint32), self.hs2[e].view(np.uint32))):
                self.mismatch += 1
        if pad:   # the row-padded layout the layer class allocates (same codes)
            w13p = padded_rows(E, 2 * I, H, torch.int8, DEV)
            w2p = padded_rows(E, H, I, torch.int8, DEV)
            w13p.copy_(self.w13)
            w2p.copy_(self.w2)
            self.w13, self.w2 = w13p, w2p


class W4Weights:
    def __init__(self, E, H, I, g, master_fn):
        self.E, self.H, self.I, self.g = E, H, I, g
        self.qw13 = torch.empty(E, 2 * I, H // 8, dtype=torch.int32, device=DEV)
        self.sc13 = torch.empty(E, 2 * I, H // g, dtype=torch.float16, device=DEV)
        self.qz13 = torch.empty(E, 2 * I // 8, H // g, dtype=torch.int32, device=DEV)
        self.qw2 = torch.empty(E, H, I // 8, dtype=torch.int32, device=DEV)
        self.sc2 = torch.empty(E, H, I // g, dtype=torch.float16, device=DEV)
        self.qz2 = torch.empty(E, H // 8, I // g, dtype=torch.int32, device=DEV)
        self.h = {k: [] for k in ("qw13", "sc13", "qz13", "qw2", "sc2", "qz2")}
        self.mismatch = 0
        for e in range(E):
            m13 = master_fn("w13", e)
            m2 = master_fn("w2", e)
            pkg.moe_quantize_weights_w4(torch.from_numpy(m13).to(DEV).view(1, 2 * I, H), g,
                                        self.qw13[e:e + 1], self.sc13[e:e + 1], self.qz13[e:e + 1])
            pkg.moe_quantize_weights_w4(torch.from_numpy(m2).to(DEV).view(1, H, I), g,
                                        self.qw2[e:e + 1], self.sc2[e:e + 1], self.qz2[e:e + 1])
            q, s, z = oracle.quantize_w4_groups(m13, g)
            self.h["qw13"].append(oracle.pack_w4_along_k(q)); self.h["sc13"].append(s)
            self.h["qz13"].append(oracle.pack_w4_along_n(z))
            q, s, z = oracle.quantize_w4_groups(m2, g)
            self.h["qw2"].append(oracle.pack_w4_along_k(q)); self.h["sc2"].append(s)
            self.h["qz2"].append(oracle.pack_w4_along_n(z))
        torch.cuda.synchronize()
        for key in self.h:
            self.h[key] = np.stack(self.h[key])
            dev = getattr(self, key).cpu()
            hv = self.h[key]
            dv = dev.numpy().view(np.uint16) if dev.dtype == torch.float16 else dev.numpy()
            hv = hv.view(np.uint16) if hv.dtype == np.float16 else hv
            if not np.array_equal(dv, hv):
                self.mismatch += 1


_CACHE = {}


def workload_weights(wl: synthetic.Workload, seed: int = 0):
    key = (wl.E, wl.H, wl.I, wl.weights, wl.group_size, seed)
    if key not in _CACHE:
        _CACHE.clear()               # keep at most one large set resident
        fn = lambda which, e: synthetic.expert_master(wl, which, e, seed)  # noqa: E731
        log(f"[weights] quantizing {wl.name}-shaped experts E={wl.E} H={wl.H} I={wl.I} ({wl.weights})")
        if wl.weights == "w8":
            _CACHE[key] = W8Weights(wl.E, wl.H, wl.I, fn, pad=True)
        else:
            _CACHE[key] = W4Weights(wl.E, wl.H, wl.I, wl.group_size, fn)
    return _CACHE[key]


def small_w8(E, H, I, seed, pad=False):
    fn = lambda which, e: synthetic.random_master((2 * I, H) if which == "w13" else (H, I),  # noqa: E731
                                                  seed * 1000 + e, tag=60 if which == "w13" else 61)
    return W8Weights(E, H, I, fn, pad=pad)


def route_both(logits: np.ndarray, k: int, renormalize: bool = True):
    """GPU router and oracle router on the same logits."""
    T, E = logits.shape
    dl = torch.from_numpy(logits).to(DEV)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    pkg.moe_route_topk(dl, k, renormalize, tw, ti)
    torch.cuda.synchronize()
    w_ref, ids_ref = oracle.route_softmax_topk(logits, k, renormalize)
    return tw, ti, w_ref, ids_ref


def run_w8_layer(W: W8Weights, x_bits, act, logits, k, renormalize=True, block_m=0, inplace=False):
    """Route + forward on the GPU; returns (gpu_out f64, ref f64, route info)."""
    T = x_bits.shape[0]
    tw, ti, w_ref, ids_ref = route_both(logits, k, renormalize)
    x = to_dev_act(x_bits, act)
    out = x if inplace else torch.empty_like(x)
    ws = torch.empty(max(pkg.moe_w8a16_workspace_bytes(T, W.H, W.I, W.E, k, block_m), 256),
                     dtype=torch.uint8, device=DEV)
    pkg.moe_w8a16_forward(x, W.w13, W.s13, W.w2, W.s2, tw, ti, out, ws, block_m)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    return got, tw.cpu().numpy(), ti.cpu().numpy(), w_ref, ids_ref


def ref_w8(W: W8Weights, x_bits, act, w_ref, ids_ref, rows=None):
    x = act_f64(x_bits, act)
    if rows is not None:
        x, w_ref, ids_ref = x[rows], w_ref[rows], ids_ref[rows]
    return oracle.moe_forward_w8(x, W.q13, W.hs13, W.q2, W.hs2, w_ref, ids_ref)


def assert_layer_close(got, ref, what):
    ok, d = oracle.layer_within_tolerance(got, ref)
    log(f"[parity] {what}: {d}")
    assert ok, f"{what}: {d}"


W8A8_FLIPS = 4   # intermediate code steps allowed per assignment (see assert_w8a8_close)


def assert_w8a8_close(got, ref, x64, W, w_ref, ids_ref, what, weight_on_input=False, num_shared=0):
    """W8A8 parity.  The layer tolerance holds up to steps of the quantized intermediate: the GPU
    computes a in fp32, the oracle in fp64, so a code whose value sits within that rounding of a half
    step can round to the neighbouring code on one side.  One step of code i moves y[h] by
    sa * W2[h, i]; W8A8_FLIPS such steps per assignment are allowed on top of the layer tolerance:
    |gpu - ref| <= 2e-2 |ref| + 1e-3 + sum_j w_j * sa_j * W8A8_FLIPS * max_i |W2_e[h, i]|."""
    sa = oracle.moe_w8a8_intermediate_scales(x64, W.q13, W.hs13, w_ref, ids_ref, weight_on_input, num_shared)
    T, H = ref.shape
    E = W.q2.shape[0]
    ids = np.asarray(ids_ref).reshape(T, -1)
    w = np.asarray(w_ref, np.float64).reshape(T, -1)
    if num_shared:
        ids = np.where((ids >= 0) & (ids < E - num_shared), ids, -1)
        w, ids = oracle.with_shared_experts(w, ids, E - num_shared, num_shared)
    if weight_on_input:
        w = np.ones_like(w)
    w2max = np.abs(W.q2.astype(np.float64)).max(axis=2) * W.hs2.astype(np.float64)      # [E, H]
    allow = np.zeros((T, H))
    for t in range(T):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if 0 <= e < E:
                allow[t] += abs(w[t, j]) * sa[t, j] * W8A8_FLIPS * w2max[e]
    d = np.abs(got - ref)
    base = 2e-2 * np.abs(ref) + 1e-3
    ok = bool(np.all(d <= base + allow)) and d.max() <= 2e-2 * np.abs(ref).max()
    n_allow = int((d > base).sum())
    log(f"[parity] {what}: max|d| {d.max():.3g} (max|ref| {np.abs(ref).max():.3g}), {n_allow} of {d.size} "
        f"elements inside the code-step allowance only, worst {float((d / (base + allow)).max()):.3f}")
    assert ok, f"{what}: max|d| {d.max()}, worst ratio {(d / (base + allow)).max()}"
