"""Seeded synthetic inputs for the weight-only-quantized MoE layer.

This module draws the random inputs that both the HIP path and the CPU
oracle consume: activations, router logits and fp32 master weights.  It holds
none of the layer's arithmetic (no quantization, routing, alignment or GEMM);
it only fixes the distributions and shapes of the workloads and hands out the
same bytes to whoever asks.

Streams: ``numpy.random.default_rng([seed, tag, expert])`` with tags
1 = activations, 2 = router logits, 3 = per-expert logit bias,
4 = w13 master of one expert, 5 = w2 master of one expert.

Workloads (shapes follow the experts_int8 page, ``create_weights``:
``w13 [E, 2I, H]``, ``w2 [E, H, I]``; the W4A16 shapes follow the moe_wna16
page, ``create_weights``):

* ``tiny``            E=8,   k=2, H=256,  I=512,   bf16
* ``mixtral_decode``  E=8,   k=2, H=4096, I=14336, bf16, T in {1, 8, 32, 64}
* ``mixtral_prefill`` as above, T in {1024, 4096}, logits + N(0, 0.5) bias per expert
* ``fine_grained``    E=64,  k=6, H=2048, I=1408,  bf16, Zipf bias 1.5*ln(1/(e+1))
* ``w4a16``           E=128, k=8, H=2048, I=768,   fp16, uint4 groups of 128
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

TAG_X, TAG_LOGITS, TAG_BIAS, TAG_W13, TAG_W2 = 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Workload:
    name: str
    E: int
    k: int
    H: int
    I: int
    act: str                 # "bf16" or "fp16"
    tokens: tuple            # token counts the workload is run at
    bias: str = "none"       # "none" | "normal0.5" | "zipf1.5"
    weights: str = "w8"      # "w8" (per-channel int8) | "w4" (uint4 groups)
    group_size: int = 128
    renormalize: bool = True
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 8, 2, 256, 512, "bf16", (16,)),
    "mixtral_decode": Workload("mixtral_decode", 8, 2, 4096, 14336, "bf16", (1, 8, 32, 64)),
    "mixtral_prefill": Workload("mixtral_prefill", 8, 2, 4096, 14336, "bf16", (1024, 4096),
                                bias="normal0.5"),
    "fine_grained": Workload("fine_grained", 64, 6, 2048, 1408, "bf16", (16, 512),
                             bias="zipf1.5"),
    "w4a16": Workload("w4a16", 128, 8, 2048, 768, "fp16", (8, 256), weights="w4"),
}

WEIGHT_STD = np.float32(0.02)


def _rng(seed, tag, e=None):
    key = [int(seed), int(tag)] if e is None else [int(seed), int(tag), int(e)]
    return np.random.default_rng(key)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round half to even) and return the uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    # NaN stays a quiet NaN
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def f32_to_fp16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE half (numpy's cast is round half to even)."""
    return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)


def activations(wl: Workload, T: int, seed: int = 0) -> np.ndarray:
    """Activations x[T, H] ~ N(0, 1), rounded to the workload's 16-bit type; uint16 bits."""
    z = _rng(seed, TAG_X).standard_normal((T, wl.H), dtype=np.float32)
    return f32_to_bf16_bits(z) if wl.act == "bf16" else f32_to_fp16_bits(z)


def expert_bias(wl: Workload, seed: int = 0) -> np.ndarray:
    """Per-expert logit offset that makes expert loads uneven (float32 [E])."""
    if wl.bias == "none":
        return np.zeros(wl.E, np.float32)
    if wl.bias == "normal0.5":
        return _rng(seed, TAG_BIAS).standard_normal(wl.E, dtype=np.float32) * np.float32(0.5)
    if wl.bias == "zipf1.5":
        rank = np.arange(1, wl.E + 1, dtype=np.float64)
        return (1.5 * np.log(1.0 / rank)).astype(np.float32)
    raise ValueError(wl.bias)


def router_logits(wl: Workload, T: int, seed: int = 0) -> np.ndarray:
    """Router logits[T, E] float32: N(0, 1) plus the workload's per-expert bias."""
    z = _rng(seed, TAG_LOGITS).standard_normal((T, wl.E), dtype=np.float32)
    return (z + expert_bias(wl, seed)[None, :]).astype(np.float32)


def expert_master(wl: Workload, which: str, e: int, seed: int = 0) -> np.ndarray:
    """fp32 master weight of one expert, N(0, 0.02): w13 -> [2I, H] (gate rows, then up rows), w2 -> [H, I]."""
    if which == "w13":
        shape, tag = (2 * wl.I, wl.H), TAG_W13
    elif which == "w2":
        shape, tag = (wl.H, wl.I), TAG_W2
    else:
        raise ValueError(which)
    return _rng(seed, tag, e).standard_normal(shape, dtype=np.float32) * WEIGHT_STD


def random_master(shape, seed: int, tag: int = 99) -> np.ndarray:
    """Generic N(0, 0.02) fp32 tensor for small ad-hoc test shapes."""
    return _rng(seed, tag).standard_normal(shape, dtype=np.float32) * WEIGHT_STD


def random_activations(T: int, H: int, act: str, seed: int, tag: int = 98) -> np.ndarray:
    z = _rng(seed, tag).standard_normal((T, H), dtype=np.float32)
    return f32_to_bf16_bits(z) if act == "bf16" else f32_to_fp16_bits(z)


def random_logits(T: int, E: int, seed: int, tag: int = 97, bias=None) -> np.ndarray:
    z = _rng(seed, tag).standard_normal((T, E), dtype=np.float32)
    if bias is not None:
        z = z + np.asarray(bias, np.float32)[None, :]
    return z.astype(np.float32)
