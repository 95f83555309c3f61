"""CPU oracle for the weight-only-quantized fused MoE layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never calls it, and this module imports nothing from
the product package.

Everything here is a plain, slow, obviously correct restatement of what the
pages define:

* experts_int8 page (vllm ... quantization.experts_int8):
  ``quantize_in_place_and_get_scales`` (per-row symmetric int8),
  ``ExpertsInt8MoEMethod.create_weights`` (w13 [E, 2I, H] int8 with the gate
  rows first and the up rows second, w2 [E, H, I] int8, fp32 scales [E, 2I]
  and [E, H]), ``quantizing_weight_loader`` (gate -> w13 rows 0..I-1,
  up -> rows I..2I-1, per output channel scales) and ``apply`` (softmax top-k
  routing through ``select_experts``, then ``fused_experts`` with
  activation "silu", ``apply_router_weight_on_input=False``).
* moe_wna16 page (vllm ... quantization.moe_wna16): ``MoeWNA16Method.create_weights``
  (packed 4-bit weights along K, group scales [E, N, K/g], packed zeros along N)
  and the weight loader's zero convention (the stored zero is the true zero).

Floating point: fp64, except where a float decides an integer code (the
quantizers); there the arithmetic is fp32 with IEEE division and round half to
even, as the page's in-place ops on an fp32 tensor compute it.

Readings where the pages are silent (the router body, the align step, the
W4 quantizer) are stated at each function.
"""
from __future__ import annotations

import itertools

import numpy as np

# ---------------------------------------------------------------------------
# 16-bit activation decoding
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly (bf16 is the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE half bit patterns (uint16) -> float64, exactly."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def act_bits_to_f64(bits: np.ndarray, act: str) -> np.ndarray:
    if act == "bf16":
        return bf16_bits_to_f64(bits)
    if act == "fp16":
        return fp16_bits_to_f64(bits)
    raise ValueError(act)


# ---------------------------------------------------------------------------
# a1: per-output-channel symmetric int8 quantizer
# ---------------------------------------------------------------------------


def quantize_int8_rows(w: np.ndarray):
    """Per-row symmetric int8 quantization of an fp32 matrix (rows = output channels).

    experts_int8 page, ``quantize_in_place_and_get_scales``: the scale of a row is
    its largest magnitude divided by the int8 maximum (127); the row is divided
    by that scale, rounded (half to even) and clamped to [-127, 127].  All of
    it runs in the tensor's own dtype, fp32 here.

    Reading for an all-zero row (the page would divide 0 by 0): scale 0, codes 0.

    Returns (q int8 [..., N, K], s float32 [..., N]).
    """
    w = np.asarray(w, dtype=np.float32)
    vmax = np.float32(127.0)
    m = np.max(np.abs(w), axis=-1, keepdims=True)            # fp32, exact
    s = (m / vmax).astype(np.float32)                         # fp32 IEEE divide
    zero = s == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (w / np.where(zero, np.float32(1.0), s)).astype(np.float32)   # fp32 IEEE divide
    r = np.rint(r)                                            # round half to even
    r = np.clip(r, -vmax, vmax)
    r = np.where(zero, np.float32(0.0), r)
    return r.astype(np.int8), s[..., 0]


def dequant_int8_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W = q * s per output channel, exactly in fp64 (an 8-bit times a 24-bit significand fits in 53 bits)."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[..., None]


# ---------------------------------------------------------------------------
# a2: softmax top-k router
# ---------------------------------------------------------------------------


def route_softmax_topk(logits: np.ndarray, k: int, renormalize: bool = True):
    """Softmax scoring, top-k selection and optional renormalisation.

    experts_int8 page, ``ExpertsInt8MoEMethod.apply``: ``select_experts`` is called
    with ``scoring_func="softmax"``, ``top_k`` and ``renormalize``; its body is not
    on the pages.  Reading: the softmax over all E experts is taken in fp64; the k
    experts with the largest fp32 logits are chosen (the same set as the largest
    probabilities, decided by exact comparisons of the inputs), listed in
    descending order, equal logits broken toward the lower expert id.  With
    ``renormalize`` the k chosen probabilities are divided by their sum.

    Returns (weights float64 [T, k], ids int32 [T, k]).
    """
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    # stable sort on the negated fp32 logits: descending, ties keep the lower id first
    ids = np.argsort(-l32, axis=1, kind="stable")[:, :k].astype(np.int32)
    l = l32.astype(np.float64)
    m = np.max(l, axis=1, keepdims=True)
    ex = np.exp(l - m)
    p = ex / np.sum(ex, axis=1, keepdims=True)
    w = np.take_along_axis(p, ids, axis=1)
    if renormalize:
        w = w / np.sum(w, axis=1, keepdims=True)
    return w, ids


def route_select(logits: np.ndarray, k: int, renormalize: bool = True, scoring: str = "softmax",
                 num_expert_group: int = 0, topk_group: int = 0, bias=None,
                 routed_scaling_factor: float = 1.0):
    """Routing with the options ``select_experts`` takes on the pages: scoring function,
    grouped top-k, a score-correction bias and a routed scaling factor.

    experts_int8 page, ``ExpertsInt8MoEMethod.apply`` (``use_grouped_topk``, ``topk_group``,
    ``num_expert_group``, ``scoring_func``, ``e_score_correction_bias``); moe_wna16 page,
    ``MoeWNA16Method.apply_monolithic`` (``routed_scaling_factor``).  The bodies are not on the
    pages; the reading used here, in order:

    1. score s_e: softmax over the E logits, or sigmoid of each logit (fp64).
    2. choice key c_e: with no bias, the fp32 logit (both scores increase with the logit, so the
       order is the same and is decided exactly); with a bias, fp32(s_e) + fp32(bias_e) added in
       fp32 (the score is rounded to fp32 first: the same precision on every side that decides).
    3. with G = num_expert_group > 1 groups of E/G consecutive experts: a group's key is the
       largest c_e in it; the topk_group groups with the largest keys (equal keys: lower group
       id) stay, the experts of the others are out.
    4. the k experts with the largest c_e among those left, descending, equal keys by lower id.
    5. weights: the unbiased scores s of the chosen experts, divided by their sum when
       renormalize, then multiplied by routed_scaling_factor.

    Returns (weights float64 [T, k], ids int32 [T, k]).
    """
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("k must be in [1, E]")
    l = l32.astype(np.float64)
    if scoring == "softmax":
        ex = np.exp(l - np.max(l, axis=1, keepdims=True))
        s = ex / np.sum(ex, axis=1, keepdims=True)
    elif scoring == "sigmoid":
        s = 1.0 / (1.0 + np.exp(-l))
    else:
        raise ValueError(f"scoring {scoring!r}")
    if bias is None:
        key = l32
    else:
        key = (s.astype(np.float32) + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    eligible = np.ones((T, E), bool)
    G = int(num_expert_group)
    if G > 1:
        if E % G or not 1 <= topk_group <= G:
            raise ValueError("E must split into num_expert_group groups and 1 <= topk_group <= groups")
        if k > topk_group * (E // G):
            raise ValueError("k is larger than the experts of the kept groups")
        gkey = key.reshape(T, G, E // G).max(axis=2)
        keep = np.argsort(-gkey, axis=1, kind="stable")[:, :topk_group]
        gmask = np.zeros((T, G), bool)
        np.put_along_axis(gmask, keep, True, axis=1)
        eligible = np.repeat(gmask, E // G, axis=1)
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        cand = np.nonzero(eligible[t])[0]                         # ascending ids
        order = np.argsort(-key[t, cand], kind="stable")          # descending key, lower id first
        ids[t] = cand[order[:k]]
    w = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / np.sum(w, axis=1, keepdims=True)
    return w * float(routed_scaling_factor), ids


# ---------------------------------------------------------------------------
# a3: token -> expert align (histogram, prefix scan, padded-block permutation)
# ---------------------------------------------------------------------------


def align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    """Rows reserved for the padded permutation: at most min(E, T*k) experts are
    non-empty and each pads to a multiple of block_m, so the number of blocks is
    at most floor((T*k + min(E, T*k)*(block_m-1)) / block_m)."""
    tk = T * k
    if tk == 0:
        return 0
    return ((tk + min(E, tk) * (block_m - 1)) // block_m) * block_m


def align_block(topk_ids: np.ndarray, E: int, block_m: int):
    """Group the flat assignments f = t*k + j by expert into padded blocks.

    Not on the pages (the fused kernel that consumes it is only called, on the
    experts_int8 page, ``apply``).  Reading: experts in ascending id; inside an
    expert the flat indices ascend (a stable order); each expert's list is padded
    with the sentinel T*k up to a multiple of block_m; experts without tokens get
    no block; ids outside [0, E) are dropped.  Every row of the capacity that is
    not part of a block holds the sentinel, every block past the last holds -1.

    Returns (sorted_ids int32 [cap], block_expert int32 [cap/block_m], num_padded int).
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    tk = ids.size
    cap = align_capacity(1, tk, E, block_m)
    sorted_ids = np.full(cap, tk, dtype=np.int32)
    block_expert = np.full(cap // block_m if block_m else 0, -1, dtype=np.int32)
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E)
    padded = -(-counts // block_m) * block_m
    off = np.concatenate([[0], np.cumsum(padded)])
    for e in range(E):
        rows = np.nonzero(ids == e)[0]                       # ascending flat index
        sorted_ids[off[e]:off[e] + rows.size] = rows
        block_expert[off[e] // block_m:off[e + 1] // block_m] = e
    return sorted_ids, block_expert, int(off[E])


def align_block_bruteforce(topk_ids, E: int, block_m: int):
    """Pure-Python loops restating the same definition (small inputs only)."""
    ids = [int(v) for v in np.asarray(topk_ids).reshape(-1)]
    tk = len(ids)
    cap = align_capacity(1, tk, E, block_m) if tk else 0
    out, be = [], []
    for e in range(E):
        mine = [f for f in range(tk) if ids[f] == e]
        if not mine:
            continue
        nb = (len(mine) + block_m - 1) // block_m
        out += mine + [tk] * (nb * block_m - len(mine))
        be += [e] * nb
    num_padded = len(out)
    out += [tk] * (cap - len(out))
    be += [-1] * (cap // block_m - len(be)) if block_m else []
    return np.array(out, np.int32), np.array(be, np.int32), num_padded


# ---------------------------------------------------------------------------
# a4 - a6: layer forward
# ---------------------------------------------------------------------------


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g / (1 + exp(-g)) (activation "silu" of ``fused_experts``)."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def moe_forward_dense(x: np.ndarray, w13_of, w2_of, topk_w: np.ndarray, topk_ids: np.ndarray,
                      I: int, weight_on_input: bool = False) -> np.ndarray:
    """Routed MoE layer with dense fp64 expert weights.

    experts_int8 page, ``ExpertsInt8MoEMethod.apply`` and ``create_weights``: for
    every assignment (t, j) of token t to expert e = topk_ids[t, j]:
    h = W13[e] x_t (rows 0..I-1 are the gate projection, rows I..2I-1 the up
    projection, ``quantizing_weight_loader``), a = silu(h_gate) * h_up,
    y = W2[e] a, and out_t = sum_j topk_w[t, j] * y (the routing weight multiplies
    the expert output: ``apply_router_weight_on_input=False``).  With
    ``weight_on_input`` (``apply_router_weight_on_input=True``) the weight
    multiplies the expert's input instead: out_t = sum_j FFN_e(topk_w[t, j] * x_t).
    Ids outside [0, E) contribute nothing.

    x: float64 [T, H]; w13_of(e) -> float64 [2I, H]; w2_of(e) -> float64 [H, I].
    Returns float64 [T, H].
    """
    x = np.asarray(x, np.float64)
    T, H = x.shape
    ids = np.asarray(topk_ids).reshape(T, -1)
    w = np.asarray(topk_w, np.float64).reshape(T, -1)
    out = np.zeros((T, H), np.float64)
    for e in np.unique(ids):
        e = int(e)
        t_idx, j_idx = np.nonzero(ids == e)
        if t_idx.size == 0:
            continue
        W13 = w13_of(e)
        W2 = w2_of(e)
        if W13 is None or W2 is None:      # expert not present (id out of range)
            continue
        wt = w[t_idx, j_idx][:, None]
        xin = wt * x[t_idx] if weight_on_input else x[t_idx]
        hmat = xin @ W13.T                 # [n, 2I]
        a = silu(hmat[:, :I]) * hmat[:, I:]
        y = a @ W2.T                       # [n, H]
        np.add.at(out, t_idx, y if weight_on_input else wt * y)
    return out


def combine_topk(y_parts: np.ndarray, topk_w: np.ndarray, topk_ids: np.ndarray, E: int) -> np.ndarray:
    """Routing-weighted combine of the experts' outputs.

    experts_int8 page, ``ExpertsInt8MoEMethod.apply`` (``fused_experts`` with
    ``apply_router_weight_on_input=False``): out_t = sum_j topk_w[t, j] * y_(t, j), where
    y_(t, j) is the output of expert topk_ids[t, j] for token t, and ids outside [0, E)
    contribute nothing.  Reading: the second product may be cut along its contraction
    (I) into parts, so y_(t, j) = sum_s y_parts[s, t*k + j] (flat assignment index t*k + j,
    the order of topk_ids.reshape(-1)).

    y_parts: [splits, T*k, H]; topk_w, topk_ids: [T, k].  Returns float64 [T, H].
    """
    y = np.asarray(y_parts, np.float64)
    ids = np.asarray(topk_ids)
    T, k = ids.shape
    w = np.asarray(topk_w, np.float64)
    out = np.zeros((T, y.shape[2]), np.float64)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E:
                out[t] += w[t, j] * y[:, t * k + j, :].sum(axis=0)
    return out


def with_shared_experts(topk_w: np.ndarray, topk_ids: np.ndarray, E: int, num_shared: int):
    """Routing extended by shared experts.

    moe_wna16 page, ``MoeWNA16Method.apply`` (``shared_experts``, ``shared_experts_input``): the
    shared experts' output is added to the routed experts' output for every token.  Reading: the
    S shared experts are gated MLPs of the routed experts' shape, stored after them (expert slots
    E .. E+S-1), that every token takes with weight 1 (a shared MLP of intermediate size S*I is
    S such experts, its intermediate split in S consecutive parts).  Returns the [T, k+S] weights
    and ids to pass to the forward.
    """
    T, k = np.asarray(topk_ids).shape
    ids = np.concatenate([np.asarray(topk_ids, np.int64),
                          np.broadcast_to(np.arange(E, E + num_shared, dtype=np.int64), (T, num_shared))], axis=1)
    w = np.concatenate([np.asarray(topk_w, np.float64), np.ones((T, num_shared))], axis=1)
    return w, ids.astype(np.int32)


def _extend_routing(topk_w, topk_ids, E_total: int, num_shared: int):
    """Routing over weight tensors of E_total experts whose last num_shared are shared experts:
    routed ids outside the routed range are dropped (id -1), the shared experts appended."""
    if not num_shared:
        return topk_w, topk_ids
    routed = np.asarray(topk_ids)
    routed = np.where((routed >= 0) & (routed < E_total - num_shared), routed, -1)
    return with_shared_experts(topk_w, routed, E_total - num_shared, num_shared)


def moe_forward_w8(x: np.ndarray, q13: np.ndarray, s13: np.ndarray, q2: np.ndarray, s2: np.ndarray,
                   topk_w: np.ndarray, topk_ids: np.ndarray, weight_on_input: bool = False,
                   num_shared: int = 0) -> np.ndarray:
    """The W8A16 layer: dequantize each used expert exactly in fp64 (W = q*s), then ``moe_forward_dense``.

    The weight tensors hold the routed experts and, after them, ``num_shared`` shared experts
    (``with_shared_experts``); topk_ids index the routed ones.  With shared experts and
    ``weight_on_input`` the shared experts take the input unscaled (weight 1)."""
    E = q13.shape[0]
    I = q13.shape[1] // 2
    topk_w, topk_ids = _extend_routing(topk_w, topk_ids, E, num_shared)

    def w13_of(e):
        return dequant_int8_rows(q13[e], s13[e]) if 0 <= e < E else None

    def w2_of(e):
        return dequant_int8_rows(q2[e], s2[e]) if 0 <= e < E else None

    return moe_forward_dense(x, w13_of, w2_of, topk_w, topk_ids, I, weight_on_input)


def moe_expert_intermediate(x: np.ndarray, W13: np.ndarray, I: int) -> np.ndarray:
    """a = silu(x W13_gate^T) * (x W13_up^T) for rows x [n, H] (fp64)."""
    hmat = np.asarray(x, np.float64) @ W13.T
    return silu(hmat[:, :I]) * hmat[:, I:]


# ---------------------------------------------------------------------------
# a7: group-wise asymmetric 4-bit weights with zero points
# ---------------------------------------------------------------------------


def f32_to_f16_rne(a) -> np.ndarray:
    return np.asarray(a, np.float32).astype(np.float16)


def quantize_w4_groups(w: np.ndarray, group_size: int):
    """Asymmetric uint4 quantization per (output row, group of K).

    The moe_wna16 page loads GPTQ/AWQ checkpoints and prints no quantizer; the
    reading used here: for each row n and group g of ``group_size`` consecutive K,
    lo = min(min w, 0), hi = max(max w, 0); the scale is (hi - lo) / 15 in fp32,
    rounded to fp16; with that fp16 scale s (as fp32): zero z = clamp(rne(-lo / s), 0, 15)
    and code q = clamp(rne(w / s) + z, 0, 15).  If the fp16 scale is 0 (a flat
    group), s = 1.  The dequantized weight is (q - z) * s (the stored zero is the
    true zero: moe_wna16 page, weight loader, GPTQ zeros get +1 to match AWQ).

    w: float32 [..., N, K].  Returns (q uint8 [..., N, K], s float16 [..., N, K/g],
    z uint8 [..., N, K/g]).
    """
    w = np.asarray(w, np.float32)
    *lead, N, K = w.shape
    if K % group_size:
        raise ValueError("K must be a multiple of group_size")
    G = K // group_size
    wg = w.reshape(*lead, N, G, group_size)
    lo = np.minimum(wg.min(axis=-1), np.float32(0.0))
    hi = np.maximum(wg.max(axis=-1), np.float32(0.0))
    s32 = ((hi - lo) / np.float32(15.0)).astype(np.float32)
    s16 = f32_to_f16_rne(s32)
    s = s16.astype(np.float32)
    flat = s == 0
    s = np.where(flat, np.float32(1.0), s)
    s16 = np.where(flat, np.float16(1.0), s16)
    z = np.clip(np.rint((-lo / s).astype(np.float32)), 0, 15)
    qf = np.rint((wg / s[..., None]).astype(np.float32)) + z[..., None]
    q = np.clip(qf, 0, 15).astype(np.uint8).reshape(*lead, N, K)
    return q, s16.astype(np.float16), z.astype(np.uint8)


def pack_w4_along_k(q: np.ndarray) -> np.ndarray:
    """uint4 codes [..., N, K] -> int32 [..., N, K/8] with code k at bits 4*(k mod 8).

    Byte-identical to the moe_wna16 page's canonical uint8 layout (two codes per
    byte along K, the even one in the low nibble) read as little-endian int32.
    """
    q = np.asarray(q, np.uint32)
    *lead, N, K = q.shape
    qq = q.reshape(*lead, N, K // 8, 8)
    word = np.zeros((*lead, N, K // 8), np.uint32)
    for i in range(8):
        word |= qq[..., i] << np.uint32(4 * i)
    return word.view(np.int32)


def unpack_w4_along_k(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed).view(np.uint32)
    *lead, N, KW = p.shape
    out = np.zeros((*lead, N, KW, 8), np.uint8)
    for i in range(8):
        out[..., i] = (p >> np.uint32(4 * i)) & 0xF
    return out.reshape(*lead, N, KW * 8)


def pack_w4_along_n(z: np.ndarray) -> np.ndarray:
    """uint4 zeros [..., N, G] -> int32 [..., N/8, G] with row n at bits 4*(n mod 8)
    (moe_wna16 page, ``create_weights``: zeros are packed along the output dimension)."""
    z = np.asarray(z, np.uint32)
    *lead, N, G = z.shape
    zz = z.reshape(*lead, N // 8, 8, G)
    word = np.zeros((*lead, N // 8, G), np.uint32)
    for i in range(8):
        word |= zz[..., i, :] << np.uint32(4 * i)
    return word.view(np.int32)


def unpack_w4_along_n(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed).view(np.uint32)
    *lead, NW, G = p.shape
    out = np.zeros((*lead, NW, 8, G), np.uint8)
    for i in range(8):
        out[..., i, :] = (p >> np.uint32(4 * i)) & 0xF
    return out.reshape(*lead, NW * 8, G)


def dequant_w4(qweight: np.ndarray, scales: np.ndarray, qzeros: np.ndarray, group_size: int) -> np.ndarray:
    """W[n, k] = (q[n, k] - z[n, k // g]) * s[n, k // g], exactly in fp64 (one expert)."""
    q = unpack_w4_along_k(qweight).astype(np.float64)
    z = unpack_w4_along_n(qzeros).astype(np.float64)
    s = np.asarray(scales, np.float16).astype(np.float64)
    zk = np.repeat(z, group_size, axis=-1)
    sk = np.repeat(s, group_size, axis=-1)
    return (q - zk) * sk


def moe_forward_w4(x: np.ndarray, qw13, s13, z13, qw2, s2, z2, group_size: int,
                   topk_w: np.ndarray, topk_ids: np.ndarray, weight_on_input: bool = False,
                   num_shared: int = 0) -> np.ndarray:
    """The W4A16 layer: per used expert, dense fp64 dequantization, then ``moe_forward_dense``
    (options as ``moe_forward_w8``)."""
    E = qw13.shape[0]
    I = qw13.shape[1] // 2
    topk_w, topk_ids = _extend_routing(topk_w, topk_ids, E, num_shared)

    def w13_of(e):
        return dequant_w4(qw13[e], s13[e], z13[e], group_size) if 0 <= e < E else None

    def w2_of(e):
        return dequant_w4(qw2[e], s2[e], z2[e], group_size) if 0 <= e < E else None

    return moe_forward_dense(x, w13_of, w2_of, topk_w, topk_ids, I, weight_on_input)


# ---------------------------------------------------------------------------
# W8A8: int8 weights with int8 activations quantized per token
# ---------------------------------------------------------------------------
# fused_moe oracle/int8 page, ``select_int8_moe_backend``: the int8 MoE kernels' default keys
# are static per-channel symmetric int8 weights (``kInt8StaticChannelSym``, the experts_int8
# weights above) and dynamic per-token symmetric int8 activations (``kInt8DynamicTokenSym``).
# The activation quantizer is not printed; reading: the per-row rule of the weights
# (``quantize_in_place_and_get_scales``) applied to every token row of the GEMM's input, in
# fp32: GEMM1's input x and GEMM2's input a = silu(h_gate) * h_up, one row per assignment.


def quantize_act_int8_rows(a) -> tuple:
    """Dynamic per-token symmetric int8 codes of the rows of a (any float dtype, taken to fp32):
    scale = max|row| / 127, code = clamp(rint(row / scale), -127, 127) in fp32; a zero row gets
    scale 0 and codes 0 (``quantize_int8_rows``)."""
    return quantize_int8_rows(np.asarray(a, np.float64).astype(np.float32))


def _w8a8_expert_rows(xin, q13e, s13e, I):
    """GEMM1 of one expert on int8 input codes and the quantized intermediate: (a8, sa)."""
    xq, sx = quantize_act_int8_rows(xin)
    acc1 = xq.astype(np.int64) @ q13e.astype(np.int64).T                        # exact
    h = acc1.astype(np.float64) * sx.astype(np.float64)[:, None] * np.asarray(s13e, np.float64)[None, :]
    a = silu(h[:, :I]) * h[:, I:]
    return quantize_act_int8_rows(a)


def moe_w8a8_intermediate_scales(x, q13, s13, topk_w, topk_ids, weight_on_input=False, num_shared=0):
    """The per-assignment scales sa of the quantized intermediate in ``moe_forward_w8a8``, as [T, k + S]
    (0 for dropped ids): one step of an intermediate code moves y by sa * W2[:, i]."""
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    E = q13.shape[0]
    I = q13.shape[1] // 2
    w, ids = _extend_routing(topk_w, topk_ids, E, num_shared)
    ids = np.asarray(ids).reshape(T, -1)
    w = np.asarray(w, np.float64).reshape(T, -1)
    out = np.zeros(ids.shape, np.float64)
    for e in np.unique(ids):
        e = int(e)
        if not 0 <= e < E:
            continue
        t_idx, j_idx = np.nonzero(ids == e)
        xin = (w[t_idx, j_idx][:, None] * x[t_idx]).astype(np.float32) if weight_on_input else x[t_idx]
        out[t_idx, j_idx] = _w8a8_expert_rows(xin, q13[e], s13[e], I)[1]
    return out


def moe_forward_w8a8(x, q13, s13, q2, s2, topk_w, topk_ids, weight_on_input=False, num_shared=0):
    """The W8A8 layer: per assignment (t, e) with weight w,
    x8, sx = quant(x_t) (or quant(w x_t) with ``weight_on_input``, w x_t rounded to fp32 first);
    h = sx * s13[e] * (q13[e] x8) (exact integer sums); a = silu(h_gate) * h_up;
    a8, sa = quant(fp32(a)); y = sa * s2[e] * (q2[e] a8); out_t += w y (1 with ``weight_on_input``).
    fp64 apart from the two quantizations.  Options as ``moe_forward_w8``."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    E = q13.shape[0]
    I = q13.shape[1] // 2
    w, ids = _extend_routing(topk_w, topk_ids, E, num_shared)
    ids = np.asarray(ids).reshape(T, -1)
    w = np.asarray(w, np.float64).reshape(T, -1)
    out = np.zeros((T, H), np.float64)
    for e in np.unique(ids):
        e = int(e)
        if not 0 <= e < E:
            continue
        t_idx, j_idx = np.nonzero(ids == e)
        wt = w[t_idx, j_idx][:, None]
        xin = (wt * x[t_idx]).astype(np.float32) if weight_on_input else x[t_idx]
        aq, sa = _w8a8_expert_rows(xin, q13[e], s13[e], I)
        acc2 = aq.astype(np.int64) @ q2[e].astype(np.int64).T
        y = acc2.astype(np.float64) * sa.astype(np.float64)[:, None] * np.asarray(s2[e], np.float64)[None, :]
        np.add.at(out, t_idx, y if weight_on_input else wt * y)
    return out


# ---------------------------------------------------------------------------
# Weight-only fp8 (OCP e4m3fn) experts with per-tensor scales
# ---------------------------------------------------------------------------
# fp8 page (vllm ... quantization.fp8): ``Fp8MoEMethod.create_weights`` (w13 [E, 2I, H] and
# w2 [E, H, I] in float8_e4m3fn, scales w13 [E, 2] (one per shard) and w2 [E]),
# ``process_weights_after_loading`` (a 16-bit checkpoint is quantized per expert with one scale
# for the merged w13 and one for w2; an fp8 checkpoint's two w13 scales are merged into their
# maximum, each shard dequantized with its own scale and quantized again with the maximum), and
# ``__init__`` (the weight-only path without fp8 activations).  ``scaled_fp8_quant`` and
# ``per_tensor_dequantize`` are only called; reading: scale = max|w| / 448 in fp32, code =
# e4m3fn(clamp(w / scale, -448, 448)) rounded to nearest even, dequant = fp32(value * scale).

E4M3_MAX = 448.0


def e4m3_round(v) -> np.ndarray:
    """fp32 values -> e4m3fn codes (uint8): clamp to [-448, 448], round to nearest even on the
    format's grid (step 2^(e-3) in binade [2^e, 2^(e+1)) for e >= -6, step 2^-9 below 2^-6); the
    sign bit is the value's (so -0 and small negatives that round to 0 give 0x80)."""
    v = np.asarray(v, np.float32).astype(np.float64)
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8)
    step = np.where(a >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
    r = np.rint(a / step) * step                        # exact: step is a power of two
    # encode the rounded magnitude
    with np.errstate(divide="ignore"):
        er = np.floor(np.log2(np.where(r > 0, r, 1.0)))
    normal = r >= 2.0 ** -6
    mant = np.where(normal, np.rint((r / 2.0 ** np.where(normal, er, 0) - 1.0) * 8), np.rint(r / 2.0 ** -9))
    bits = np.where(normal, ((er + 7).astype(np.int64) << 3) | mant.astype(np.int64), mant.astype(np.int64))
    return (bits | (sign.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """e4m3fn codes -> float64, exactly (codes 0x7F / 0xFF are NaN)."""
    b = np.asarray(codes, np.uint8).astype(np.int64)
    sgn = np.where(b & 0x80, -1.0, 1.0)
    ex = (b >> 3) & 0xF
    m = (b & 7).astype(np.float64)
    val = np.where(ex == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (ex - 7))
    val = np.where((b & 0x7F) == 0x7F, np.nan, val)
    return sgn * val


def quantize_fp8_tensor(w, scale=None):
    """``scaled_fp8_quant``: one scale for the whole tensor (dynamic: max|w| / 448 in fp32; or the
    given fp32 scale), codes e4m3fn(w / scale) (fp32 divide).  A zero tensor gets scale 0 and
    codes 0.  Returns (codes uint8, scale float32)."""
    w = np.asarray(w, np.float32)
    if scale is None:
        scale = np.float32(np.max(np.abs(w)) / np.float32(E4M3_MAX)) if w.size else np.float32(0)
    scale = np.float32(scale)
    if scale == 0:
        return np.zeros(w.shape, np.uint8), scale
    return e4m3_round((w / scale).astype(np.float32)), scale


def dequant_fp8(codes, scale) -> np.ndarray:
    """``per_tensor_dequantize``: fp32(value * scale)."""
    return (e4m3_decode(codes).astype(np.float32) * np.float32(scale)).astype(np.float32)


def fp8_merge_w13_scales(q13, s13):
    """fp8 checkpoint with one scale per w13 shard (s13 [E, 2]): per expert the larger scale is kept;
    each shard is dequantized with its own scale (fp32) and quantized again with the larger one.
    Returns (codes uint8 [E, 2I, H], scales float32 [E])."""
    q13 = np.asarray(q13, np.uint8)
    s13 = np.asarray(s13, np.float32)
    E, N2, _ = q13.shape
    I = N2 // 2
    out = np.empty_like(q13)
    smax = s13.max(axis=1).astype(np.float32)
    for e in range(E):
        for shard in range(2):
            rows = slice(shard * I, (shard + 1) * I)
            out[e, rows] = quantize_fp8_tensor(dequant_fp8(q13[e, rows], s13[e, shard]), smax[e])[0]
    return out, smax


def moe_forward_fp8(x, q13, s13, q2, s2, topk_w, topk_ids, weight_on_input=False, num_shared=0):
    """The weight-only fp8 layer: W = decode(q) * s exactly in fp64 (one scale per expert and
    matrix), then ``moe_forward_dense`` (options as ``moe_forward_w8``)."""
    E = q13.shape[0]
    I = q13.shape[1] // 2
    topk_w, topk_ids = _extend_routing(topk_w, topk_ids, E, num_shared)

    def w13_of(e):
        return e4m3_decode(q13[e]) * float(s13[e]) if 0 <= e < E else None

    def w2_of(e):
        return e4m3_decode(q2[e]) * float(s2[e]) if 0 <= e < E else None

    return moe_forward_dense(x, w13_of, w2_of, topk_w, topk_ids, I, weight_on_input)


# ---------------------------------------------------------------------------
# GPTQ / AWQ checkpoint import into the canonical 4-bit layout
# ---------------------------------------------------------------------------
# moe_wna16 page, ``MoeWNA16Method.get_weight_loader``: ``convert_awq_tensor``,
# ``convert_gptq_int4_qzeros`` and ``moe_wna16_weight_loader`` turn the packed
# int32 tensors of AWQ and GPTQ checkpoints into the page's canonical uint8
# layout (codes [N, K/2] along K, zeros [N/2, K/g] along N, even index in the
# low nibble; scales [N, K/g]); ``MoeWNA16Method.create_weights`` halves the
# group size until it divides both H and I and the loader repeats scales and
# zeros to match.  The steps below follow the loader; the last one, from the
# page's uint8 layout to this library's int32 words, is this library's own
# packing (codes: the same bytes; zeros: 8 rows of one group per word).

AWQ_REVERSE_ORDER = (0, 4, 1, 5, 2, 6, 3, 7)   # the page's reverse_awq_pack_order


def _nibbles_low_first(t: np.ndarray) -> np.ndarray:
    """int32 [a, b] -> uint8 nibbles [a, 8b]: bytes in memory order, low nibble before high."""
    b8 = np.ascontiguousarray(np.asarray(t, np.int32)).view(np.uint8)          # [a, 4b] little-endian bytes
    nib = np.stack([b8 & 0xF, b8 >> 4], axis=-1)                                # [a, 4b, 2]
    return nib.reshape(t.shape[0], -1)


def awq_to_page_uint8(t: np.ndarray, kind: str) -> np.ndarray:
    """``convert_awq_tensor``: AWQ qweight int32 [K, N/8] -> uint8 [N, K/2]; AWQ qzeros int32
    [K/g, N/8] -> uint8 [N/2, K/g].  Unpack the nibbles, undo AWQ's order inside every group of
    eight, transpose, and pack pairs again (along K for codes, along N for zeros)."""
    a = t.shape[0]
    nib = _nibbles_low_first(t).reshape(-1, 8)[:, list(AWQ_REVERSE_ORDER)].reshape(a, -1)   # [a, n]
    tt = nib.T                                                                              # [n, a]
    if kind == "qweight":
        return (tt[:, 0::2] + 16 * tt[:, 1::2]).astype(np.uint8)
    if kind == "qzeros":
        return (tt[0::2, :] + 16 * tt[1::2, :]).astype(np.uint8)
    raise ValueError(kind)


def gptq_qweight_to_page_uint8(t: np.ndarray) -> np.ndarray:
    """GPTQ qweight int32 [K/8, N] (codes packed along K) -> uint8 [N, K/2]: transpose, view bytes."""
    return np.ascontiguousarray(np.asarray(t, np.int32).T).view(np.uint8)


def gptq_qzeros_to_page_uint8(t: np.ndarray) -> np.ndarray:
    """``convert_gptq_int4_qzeros``: GPTQ qzeros int32 [K/g, N/8] store zero - 1; add 1 to each nibble
    and pack the pair again with uint8 arithmetic (a stored 15 carries into the high nibble, as the
    page's byte sum does), then transpose -> uint8 [N/2, K/g]."""
    b8 = np.ascontiguousarray(np.asarray(t, np.int32)).view(np.uint8)          # [K/g, N/2]
    lo = (b8 & 0xF).astype(np.uint8) + np.uint8(1)
    hi = (b8 >> 4).astype(np.uint8) + np.uint8(1)
    packed = (lo + hi * np.uint8(16)).astype(np.uint8)                           # wraps like uint8 tensors
    return np.ascontiguousarray(packed.T)


def wna16_group_size(H: int, I: int, group_size: int):
    """``MoeWNA16Method.create_weights``: halve the group size until it divides I and H (never below 32);
    returns (group size, factor the loaded scales and zeros are repeated by)."""
    g, f = int(group_size), 1
    while I % g or H % g:
        g //= 2
        f *= 2
        if g < 32:
            raise ValueError("group size fell below 32")
    return g, f


def repeat_groups(t: np.ndarray, factor: int) -> np.ndarray:
    """``repeat_interleave(factor, 1)`` of the loader: every group column repeated factor times."""
    return np.repeat(np.asarray(t), factor, axis=1)


def page_codes_to_words(u8: np.ndarray) -> np.ndarray:
    """uint8 codes [N, K/2] -> int32 [N, K/8]: the same bytes read as little-endian words."""
    return np.ascontiguousarray(u8).view(np.int32)


def page_zeros_to_words(u8: np.ndarray) -> np.ndarray:
    """uint8 zeros [N/2, G] (rows 2i, 2i+1 in byte i) -> int32 [N/8, G] with row n at bits 4(n mod 8)."""
    u = np.asarray(u8, np.uint32)
    N2, G = u.shape
    q = u.reshape(N2 // 4, 4, G)
    return (q[:, 0] | (q[:, 1] << 8) | (q[:, 2] << 16) | (q[:, 3] << 24)).view(np.int32)


def import_awq(qweight: np.ndarray, qzeros: np.ndarray, scales: np.ndarray, H: int, I: int, group_size: int):
    """One expert matrix of an AWQ checkpoint -> (qweight int32 [N, K/8], scales fp16 [N, K/g'],
    qzeros int32 [N/8, K/g']) in this library's layout, with the group size g' of ``wna16_group_size``.
    AWQ shapes: qweight [K, N/8], qzeros [K/g, N/8], scales [K/g, N]."""
    _, f = wna16_group_size(H, I, group_size)
    qw = page_codes_to_words(awq_to_page_uint8(qweight, "qweight"))
    qz = page_zeros_to_words(repeat_groups(awq_to_page_uint8(qzeros, "qzeros"), f))
    sc = repeat_groups(np.asarray(scales, np.float16).T, f)
    return qw, np.ascontiguousarray(sc), qz


def import_gptq(qweight: np.ndarray, qzeros: np.ndarray, scales: np.ndarray, H: int, I: int, group_size: int):
    """One expert matrix of a GPTQ checkpoint (4-bit) -> the layout of ``import_awq``.
    GPTQ shapes: qweight [K/8, N], qzeros [K/g, N/8] (zero - 1), scales [K/g, N]."""
    _, f = wna16_group_size(H, I, group_size)
    qw = page_codes_to_words(gptq_qweight_to_page_uint8(qweight))
    qz = page_zeros_to_words(repeat_groups(gptq_qzeros_to_page_uint8(qzeros), f))
    sc = repeat_groups(np.asarray(scales, np.float16).T, f)
    return qw, np.ascontiguousarray(sc), qz


# ---------------------------------------------------------------------------
# Tolerance of the layer output (floating-point result)
# ---------------------------------------------------------------------------


def layer_within_tolerance(got: np.ndarray, ref: np.ndarray, rel: float = 2e-2, abs_: float = 1e-3):
    """max|got-ref| <= rel*max|ref| and |got-ref| <= rel*|ref| + abs_ per element.

    Returns (ok, detail dict)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    lim = rel * np.abs(ref) + abs_
    bad = d > lim
    mx = float(d.max()) if d.size else 0.0
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    ok = (not bad.any()) and (mx <= rel * mref or mx == 0.0)
    return ok, {"max_abs_err": mx, "max_abs_ref": mref, "n_bad": int(bad.sum()),
                "worst_ratio": float((d / lim).max()) if d.size else 0.0}


def topk_subsets_bruteforce(logits_row: np.ndarray, k: int):
    """All k-subsets whose every member's logit is >= every non-member's logit (E small)."""
    l = np.asarray(logits_row, np.float32)
    E = l.size
    good = []
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(l[a] >= l[b] for a in sub for b in rest):
            good.append(sub)
    return good
