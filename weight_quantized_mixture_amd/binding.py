"""ctypes binding of libmoe_wq.so (the C ABI declared in include/moe_wq.h).

Argument marshalling only: every function takes torch tensors (device memory
the caller owns), passes their data pointers, sizes and the current HIP
stream to the C call of the same name, and raises on a non-zero status
(``ValueError`` for invalid arguments and workspace sizes, ``NotImplementedError``
for unsupported cases, ``RuntimeError`` for HIP failures), mirroring the
pages' error types (experts_int8 page, quantizing_weight_loader raises
ValueError; apply raises NotImplementedError).  There is no fallback: if the
library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_wq.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
MOE_BF16, MOE_FP16 = 0, 1

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size = ctypes.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_quantize_weights_int8": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "moe_route_topk": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_int, _c_p, _c_p, _c_p]),
    "moe_route_select": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "moe_align_capacity": (_c_i64, [_c_i64, _c_i64, _c_i64, _c_i64]),
    "moe_align_block": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "moe_w8a16_block_m": (_c_i64, [_c_i64] * 5),
    "moe_w8a16_workspace_bytes": (_c_size, [_c_i64] * 6),
    "moe_w8a16_forward": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                   _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                   _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w8a16_forward_noalloc": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                           _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                           _c_p, _c_p, _c_i64, _c_p, _c_p]),
    "moe_w8a16_apply": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_int,
                                 _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                 _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w4a16_apply": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_int,
                                 _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                 _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w8a16_splits": (_c_i64, [_c_i64] * 6),
    "moe_quantize_act_int8": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "moe_w8a8_workspace_bytes": (_c_size, [_c_i64] * 6 + [_c_p]),
    "moe_w8a8_forward": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                  _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                  _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w8a8_apply": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p,
                                _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_quantize_weights_fp8": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p]),
    "moe_fp8_merge_w13_scales": (_c_int, [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p]),
    "moe_wfp8a16_workspace_bytes": (_c_size, [_c_i64] * 6 + [_c_p]),
    "moe_wfp8a16_forward": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                     _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                     _c_size, _c_p]),
    "moe_wfp8a16_apply": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p,
                                   _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p,
                                   _c_size, _c_p]),
    "moe_wna16_group_size": (_c_int, [_c_i64, _c_i64, _c_i64, _c_p, _c_p]),
    "moe_w4_import": (_c_int, [_c_int, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "moe_w8a16_workspace_bytes_ex": (_c_size, [_c_i64] * 6 + [_c_p]),
    "moe_w4a16_workspace_bytes_ex": (_c_size, [_c_i64] * 6 + [_c_p]),
    "moe_w8a16_forward_ex": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                      _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w8a16_apply_ex": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p,
                                    _c_p, _c_p, _c_i64, _c_p, _c_p, _c_i64,
                                    _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w4a16_forward_ex": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                      _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                      _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w4a16_apply_ex": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p,
                                    _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                    _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
    "moe_w8a16_intermediate_bytes": (_c_size, [_c_i64] * 6),
    "moe_w8a16_requant": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_i64, _c_p]),
    "moe_w8a16_gemm1": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                 _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p, _c_i64, _c_p, _c_p]),
    "moe_w8a16_gemm2": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                 _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p]),
    "moe_combine_topk": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                  _c_p, _c_p, _c_int, _c_p, _c_p]),
    "moe_quantize_weights_w4": (_c_int, [_c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "moe_w4a16_workspace_bytes": (_c_size, [_c_i64] * 6),
    "moe_w4a16_forward": (_c_int, [_c_p, _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                   _c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                   _c_p, _c_p, _c_i64, _c_p, _c_p, _c_size, _c_p]),
}

class MoeRouting(ctypes.Structure):
    """struct moe_routing of moe_wq.h (routing options of select_experts)."""
    _fields_ = [("scoring", ctypes.c_int), ("renormalize", ctypes.c_int), ("num_expert_group", ctypes.c_int64),
                ("topk_group", ctypes.c_int64), ("e_score_correction_bias", ctypes.c_void_p),
                ("routed_scaling_factor", ctypes.c_float)]


MOE_SCORING = {"softmax": 0, "sigmoid": 1}


class MoeFusedOpts(ctypes.Structure):
    """struct moe_fused_opts of moe_wq.h (apply_router_weight_on_input, shared experts)."""
    _fields_ = [("apply_router_weight_on_input", ctypes.c_int), ("num_shared_experts", ctypes.c_int64)]

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_wq.so (built in-tree by __graft_entry__.build()); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class MoeError(RuntimeError):
    pass


def _check(status: int, name: str):
    if status == MOE_OK:
        return
    detail = lib().moe_last_error().decode(errors="replace")
    text = f"{name}: {lib().moe_status_string(status).decode()}: {detail}"
    if status in (MOE_ERR_INVALID_ARGUMENT, MOE_ERR_WORKSPACE_TOO_SMALL):
        raise ValueError(text)
    if status == MOE_ERR_UNSUPPORTED:
        raise NotImplementedError(text)
    raise MoeError(text)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _act(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float16:
        return MOE_FP16
    raise NotImplementedError(f"activation dtype {t.dtype} (bf16 or fp16 only)")


def _need_act(x, name="x"):
    """Activations: a contiguous 2-D bf16/fp16 device tensor; returns (T, H, act code)."""
    act = _act(x)
    if x.dim() != 2:
        raise ValueError(f"{name}: expected [T, H], got shape {tuple(x.shape)}")
    _need(x, x.dtype, tuple(x.shape), name)
    return x.shape[0], x.shape[1], act


def _need_align(T, k, E, block_m, sorted_ids, block_expert, num_padded):
    """The align outputs the stage calls read, sized by moe_align_capacity."""
    if block_m < 1:
        raise ValueError(f"block_m must be >= 1, got {block_m}")
    cap = moe_align_capacity(T, k, E, block_m)
    need = [(sorted_ids, (cap,), "sorted_ids"), (block_expert, (cap // block_m,), "block_expert"),
            (num_padded, (1,), "num_padded")]
    for t, shape, name in need:
        _need(t, torch.int32, shape, name, device=False)
    for t, shape, name in need:
        _need(t, torch.int32, shape, name)


def _row_stride(t, dtype, shape, name) -> int:
    """Weights may be row-padded views: [E, N, K] with strides (N*ld, ld, 1), ld >= K; returns ld."""
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    E, N, K = shape
    ld = t.stride(1)
    if t.stride(2) != 1 or ld < K or (E > 1 and t.stride(0) != N * ld):
        raise ValueError(f"{name}: needs rows of stride >= K and experts of stride N*row_stride, got {t.stride()}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return ld


def _need(t, dtype, shape, name, device=True):
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


# ---------------------------------------------------------------------------
# C calls of the same names
# ---------------------------------------------------------------------------


def moe_quantize_weights_int8(w: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, stream=None):
    E, N, K = w.shape
    _need(w, torch.float32, (E, N, K), "w")
    _need(q, torch.int8, (E, N, K), "q")
    _need(scale, torch.float32, (E, N), "scale")
    _check(lib().moe_quantize_weights_int8(_ptr(w), E, N, K, _ptr(q), _ptr(scale), _stream(stream)),
           "moe_quantize_weights_int8")


def moe_route_topk(logits: torch.Tensor, k: int, renormalize: bool, topk_w: torch.Tensor,
                   topk_ids: torch.Tensor, stream=None):
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _check(lib().moe_route_topk(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(topk_w),
                                _ptr(topk_ids), _stream(stream)), "moe_route_topk")


def routing_struct(E: int, renormalize: bool = True, scoring: str = "softmax", num_expert_group: int = 0,
                   topk_group: int = 0, e_score_correction_bias=None, routed_scaling_factor: float = 1.0):
    """A MoeRouting for the C calls; the bias (fp32 [E] device tensor) must stay alive while it is used."""
    if scoring not in MOE_SCORING:
        raise ValueError(f"scoring must be one of {sorted(MOE_SCORING)}, got {scoring!r}")
    if e_score_correction_bias is not None:
        _need(e_score_correction_bias, torch.float32, (E,), "e_score_correction_bias")
    return MoeRouting(MOE_SCORING[scoring], int(bool(renormalize)), int(num_expert_group), int(topk_group),
                      None if e_score_correction_bias is None else e_score_correction_bias.data_ptr(),
                      float(routed_scaling_factor))


def moe_route_select(logits: torch.Tensor, k: int, topk_w: torch.Tensor, topk_ids: torch.Tensor,
                     renormalize: bool = True, scoring: str = "softmax", num_expert_group: int = 0,
                     topk_group: int = 0, e_score_correction_bias=None, routed_scaling_factor: float = 1.0,
                     stream=None):
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    r = routing_struct(E, renormalize, scoring, num_expert_group, topk_group, e_score_correction_bias,
                       routed_scaling_factor)
    _check(lib().moe_route_select(_ptr(logits), T, E, k, ctypes.byref(r), _ptr(topk_w), _ptr(topk_ids),
                                  _stream(stream)), "moe_route_select")


def moe_align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return int(lib().moe_align_capacity(T, k, E, block_m))


def moe_align_block(topk_ids: torch.Tensor, E: int, block_m: int, sorted_ids: torch.Tensor,
                    block_expert: torch.Tensor, num_padded: torch.Tensor, stream=None):
    T, k = topk_ids.shape
    cap = moe_align_capacity(T, k, E, block_m)
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(sorted_ids, torch.int32, (cap,), "sorted_ids")
    _need(block_expert, torch.int32, (cap // block_m,), "block_expert")
    _need(num_padded, torch.int32, (1,), "num_padded")
    _check(lib().moe_align_block(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_ids), _ptr(block_expert),
                                 _ptr(num_padded), _stream(stream)), "moe_align_block")


def moe_w8a16_block_m(T, H, I, E, k) -> int:
    return int(lib().moe_w8a16_block_m(T, H, I, E, k))


def moe_w8a16_splits(T, H, I, E, k, block_m=0) -> int:
    return int(lib().moe_w8a16_splits(T, H, I, E, k, block_m))


def moe_w8a16_intermediate_bytes(T, H, I, E, k, block_m=0) -> int:
    return int(lib().moe_w8a16_intermediate_bytes(T, H, I, E, k, block_m))


def _need_bytes(t: torch.Tensor, nbytes: int, name: str):
    if not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: needs a contiguous buffer of at least {nbytes} bytes")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def moe_w8a16_workspace_bytes(T, H, I, E, k, block_m=0) -> int:
    return int(lib().moe_w8a16_workspace_bytes(T, H, I, E, k, block_m))


def moe_w4a16_workspace_bytes(T, H, I, E, k, block_m=0) -> int:
    return int(lib().moe_w4a16_workspace_bytes(T, H, I, E, k, block_m))


def _w8_shapes(w13, w2):
    E, N2, H = w13.shape
    I = N2 // 2
    return E, H, I


def moe_w8a16_forward(x, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, workspace,
                      block_m: int = 0, stream=None):
    """out = MoE(x) for int8 experts; `workspace` is a uint8 device tensor of
    at least moe_w8a16_workspace_bytes(...) bytes; `out` may be `x`."""
    T, H, act = _need_act(x)
    E, _, I = _w8_shapes(w13, w2)
    k = topk_ids.shape[1]
    ld13 = _row_stride(w13, torch.int8, (E, 2 * I, H), "w13")
    _need(w13_scale, torch.float32, (E, 2 * I), "w13_scale")
    ld2 = _row_stride(w2, torch.int8, (E, H, I), "w2")
    _need(w2_scale, torch.float32, (E, H), "w2_scale")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    _need_bytes(workspace, moe_w8a16_workspace_bytes(T, H, I, E, k, block_m), "workspace")
    _check(lib().moe_w8a16_forward(_ptr(x), act, T, H, I, E, k, _ptr(w13), _ptr(w13_scale), ld13,
                                   _ptr(w2), _ptr(w2_scale), ld2, _ptr(topk_w), _ptr(topk_ids), block_m,
                                   _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "moe_w8a16_forward")


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20     # size of the static workspace of moe_w8a16_forward_noalloc


def moe_w8a16_forward_noalloc(x, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, block_m: int = 0,
                              stream=None):
    """moe_w8a16_forward on the library's static device workspace (no workspace argument, nothing
    allocated); raises ValueError when the batch needs more than MOE_NOALLOC_SCRATCH_BYTES."""
    T, H, act = _need_act(x)
    E, _, I = _w8_shapes(w13, w2)
    k = topk_ids.shape[1]
    ld13 = _row_stride(w13, torch.int8, (E, 2 * I, H), "w13")
    _need(w13_scale, torch.float32, (E, 2 * I), "w13_scale")
    ld2 = _row_stride(w2, torch.int8, (E, H, I), "w2")
    _need(w2_scale, torch.float32, (E, H), "w2_scale")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    _check(lib().moe_w8a16_forward_noalloc(_ptr(x), act, T, H, I, E, k, _ptr(w13), _ptr(w13_scale), ld13,
                                           _ptr(w2), _ptr(w2_scale), ld2, _ptr(topk_w), _ptr(topk_ids), block_m,
                                           _ptr(out), _stream(stream)), "moe_w8a16_forward_noalloc")


def moe_w8a16_gemm1(x, w13, w13_scale, sorted_ids, block_expert, num_padded, block_m, k, a, stream=None):
    T, H, act = _need_act(x)
    E, N2, _ = w13.shape
    I = N2 // 2
    ld13 = _row_stride(w13, torch.int8, (E, N2, H), "w13")
    _need(w13_scale, torch.float32, (E, N2), "w13_scale")
    _need_align(T, k, E, block_m, sorted_ids, block_expert, num_padded)
    _need_bytes(a, moe_w8a16_intermediate_bytes(T, H, I, E, k, block_m), "a")
    _check(lib().moe_w8a16_gemm1(_ptr(x), act, T, H, I, E, k, _ptr(w13), _ptr(w13_scale), ld13,
                                 _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded), block_m, _ptr(a),
                                 _stream(stream)), "moe_w8a16_gemm1")


def moe_w8a16_requant(a, T, I, E, k, sorted_ids, num_padded, block_m, stream=None):
    cap = moe_align_capacity(T, k, E, block_m)
    _need(sorted_ids, torch.int32, (cap,), "sorted_ids")
    _need(num_padded, torch.int32, (1,), "num_padded")
    _need_bytes(a, moe_w8a16_intermediate_bytes(T, 128, I, E, k, block_m), "a")
    _check(lib().moe_w8a16_requant(_ptr(a), T, I, E, k, _ptr(sorted_ids), _ptr(num_padded), block_m,
                                   _stream(stream)), "moe_w8a16_requant")


def moe_w8a16_gemm2(a, T, k, w2, w2_scale, sorted_ids, block_expert, num_padded, block_m, splits, y,
                    stream=None):
    E, H, I = w2.shape
    ld2 = _row_stride(w2, torch.int8, (E, H, I), "w2")
    _need(w2_scale, torch.float32, (E, H), "w2_scale")
    _need_align(T, k, E, block_m, sorted_ids, block_expert, num_padded)
    _need_bytes(a, moe_w8a16_intermediate_bytes(T, H, I, E, k, block_m), "a")
    _need(y, torch.float32, (splits, T * k, H), "y")
    _check(lib().moe_w8a16_gemm2(_ptr(a), T, H, I, E, k, _ptr(w2), _ptr(w2_scale), ld2, _ptr(sorted_ids),
                                 _ptr(block_expert), _ptr(num_padded), block_m, splits, _ptr(y),
                                 _stream(stream)), "moe_w8a16_gemm2")


def moe_combine_topk(y, splits, topk_w, topk_ids, E, out, stream=None):
    T, H = out.shape
    k = topk_ids.shape[1]
    _need(y, torch.float32, (splits, T * k, H), "y")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need_act(out, "out")
    _check(lib().moe_combine_topk(_ptr(y), splits, T, k, H, E, _ptr(topk_w), _ptr(topk_ids), _act(out),
                                  _ptr(out), _stream(stream)), "moe_combine_topk")


def moe_quantize_weights_w4(w, group_size, qweight, scales, qzeros, stream=None):
    E, N, K = w.shape
    _need(w, torch.float32, (E, N, K), "w")
    _need(qweight, torch.int32, (E, N, K // 8), "qweight")
    _need(scales, torch.float16, (E, N, K // group_size), "scales")
    _need(qzeros, torch.int32, (E, N // 8, K // group_size), "qzeros")
    _check(lib().moe_quantize_weights_w4(_ptr(w), E, N, K, group_size, _ptr(qweight), _ptr(scales),
                                         _ptr(qzeros), _stream(stream)), "moe_quantize_weights_w4")


def moe_w4a16_forward(x, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales, w2_qzeros,
                      group_size, topk_w, topk_ids, out, workspace, block_m: int = 0, stream=None):
    T, H, act = _need_act(x)
    E, N2, _ = w13_qweight.shape
    I = N2 // 2
    k = topk_ids.shape[1]
    _need(w13_qweight, torch.int32, (E, 2 * I, H // 8), "w13_qweight")
    _need(w13_scales, torch.float16, (E, 2 * I, H // group_size), "w13_scales")
    _need(w13_qzeros, torch.int32, (E, 2 * I // 8, H // group_size), "w13_qzeros")
    _need(w2_qweight, torch.int32, (E, H, I // 8), "w2_qweight")
    _need(w2_scales, torch.float16, (E, H, I // group_size), "w2_scales")
    _need(w2_qzeros, torch.int32, (E, H // 8, I // group_size), "w2_qzeros")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    _need_bytes(workspace, moe_w4a16_workspace_bytes(T, H, I, E, k, block_m), "workspace")
    _check(lib().moe_w4a16_forward(_ptr(x), act, T, H, I, E, k, _ptr(w13_qweight), _ptr(w13_scales),
                                   _ptr(w13_qzeros), _ptr(w2_qweight), _ptr(w2_scales), _ptr(w2_qzeros),
                                   group_size, _ptr(topk_w), _ptr(topk_ids), block_m, _ptr(out),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(stream)), "moe_w4a16_forward")


def moe_w8a16_apply(x, router_logits, renormalize, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out,
                    workspace, block_m: int = 0, stream=None):
    """Route from logits and run the layer in one call; topk_w / topk_ids receive the routing."""
    T, H, act = _need_act(x)
    E, _, I = _w8_shapes(w13, w2)
    k = topk_ids.shape[1]
    _need(router_logits, torch.float32, (T, E), "router_logits")
    ld13 = _row_stride(w13, torch.int8, (E, 2 * I, H), "w13")
    _need(w13_scale, torch.float32, (E, 2 * I), "w13_scale")
    ld2 = _row_stride(w2, torch.int8, (E, H, I), "w2")
    _need(w2_scale, torch.float32, (E, H), "w2_scale")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    _need_bytes(workspace, moe_w8a16_workspace_bytes(T, H, I, E, k, block_m), "workspace")
    _check(lib().moe_w8a16_apply(_ptr(x), act, T, H, I, E, k, _ptr(router_logits), int(bool(renormalize)),
                                 _ptr(w13), _ptr(w13_scale), ld13, _ptr(w2), _ptr(w2_scale), ld2, _ptr(topk_w),
                                 _ptr(topk_ids), block_m, _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)), "moe_w8a16_apply")


def moe_w4a16_apply(x, router_logits, renormalize, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales,
                    w2_qzeros, group_size, topk_w, topk_ids, out, workspace, block_m: int = 0, stream=None):
    T, H, act = _need_act(x)
    E, N2, _ = w13_qweight.shape
    I = N2 // 2
    k = topk_ids.shape[1]
    _need(router_logits, torch.float32, (T, E), "router_logits")
    _need(w13_qweight, torch.int32, (E, 2 * I, H // 8), "w13_qweight")
    _need(w13_scales, torch.float16, (E, 2 * I, H // group_size), "w13_scales")
    _need(w13_qzeros, torch.int32, (E, 2 * I // 8, H // group_size), "w13_qzeros")
    _need(w2_qweight, torch.int32, (E, H, I // 8), "w2_qweight")
    _need(w2_scales, torch.float16, (E, H, I // group_size), "w2_scales")
    _need(w2_qzeros, torch.int32, (E, H // 8, I // group_size), "w2_qzeros")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    _need_bytes(workspace, moe_w4a16_workspace_bytes(T, H, I, E, k, block_m), "workspace")
    _check(lib().moe_w4a16_apply(_ptr(x), act, T, H, I, E, k, _ptr(router_logits), int(bool(renormalize)),
                                 _ptr(w13_qweight), _ptr(w13_scales), _ptr(w13_qzeros), _ptr(w2_qweight),
                                 _ptr(w2_scales), _ptr(w2_qzeros), group_size, _ptr(topk_w), _ptr(topk_ids),
                                 block_m, _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)), "moe_w4a16_apply")


# ---------------------------------------------------------------------------
# Layer calls with routing options (moe_routing) and fused options (moe_fused_opts)
# ---------------------------------------------------------------------------


def fused_opts(num_shared_experts: int = 0, apply_router_weight_on_input: bool = False) -> MoeFusedOpts:
    return MoeFusedOpts(int(bool(apply_router_weight_on_input)), int(num_shared_experts))


def moe_w8a16_workspace_bytes_ex(T, H, I, E, k, block_m=0, num_shared_experts=0,
                                 apply_router_weight_on_input=False) -> int:
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    return int(lib().moe_w8a16_workspace_bytes_ex(T, H, I, E, k, block_m, ctypes.byref(o)))


def moe_w4a16_workspace_bytes_ex(T, H, I, E, k, block_m=0, num_shared_experts=0,
                                 apply_router_weight_on_input=False) -> int:
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    return int(lib().moe_w4a16_workspace_bytes_ex(T, H, I, E, k, block_m, ctypes.byref(o)))


def _w8_checked(x, w13, w13_scale, w2, w2_scale, S):
    T, H, act = _need_act(x)
    Et, N2, _ = w13.shape
    I = N2 // 2
    if S < 0 or S >= Et:
        raise ValueError(f"num_shared_experts {S} must be in [0, {Et})")
    ld13 = _row_stride(w13, torch.int8, (Et, 2 * I, H), "w13")
    _need(w13_scale, torch.float32, (Et, 2 * I), "w13_scale")
    ld2 = _row_stride(w2, torch.int8, (Et, H, I), "w2")
    _need(w2_scale, torch.float32, (Et, H), "w2_scale")
    return T, H, I, Et - S, act, ld13, ld2


def moe_w8a16_forward_ex(x, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, workspace, num_shared_experts=0,
                         apply_router_weight_on_input=False, block_m: int = 0, stream=None):
    """moe_w8a16_forward with shared experts (the last `num_shared_experts` of the weight tensors) and
    the routing weight optionally applied to the input; topk_ids index the routed experts."""
    T, H, I, E, act, ld13, ld2 = _w8_checked(x, w13, w13_scale, w2, w2_scale, num_shared_experts)
    k = topk_ids.shape[1]
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_w8a16_workspace_bytes_ex(T, H, I, E, k, block_m, num_shared_experts,
                                                        apply_router_weight_on_input), "workspace")
    _check(lib().moe_w8a16_forward_ex(_ptr(x), act, T, H, I, E, k, _ptr(w13), _ptr(w13_scale), ld13, _ptr(w2),
                                      _ptr(w2_scale), ld2, _ptr(topk_w), _ptr(topk_ids), ctypes.byref(o), block_m,
                                      _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "moe_w8a16_forward_ex")


def moe_w8a16_apply_ex(x, router_logits, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, workspace,
                       renormalize=True, scoring="softmax", num_expert_group=0, topk_group=0,
                       e_score_correction_bias=None, routed_scaling_factor=1.0, num_shared_experts=0,
                       apply_router_weight_on_input=False, block_m: int = 0, stream=None):
    """Route from logits with the select_experts options, then the layer with the fused options."""
    T, H, I, E, act, ld13, ld2 = _w8_checked(x, w13, w13_scale, w2, w2_scale, num_shared_experts)
    k = topk_ids.shape[1]
    _need(router_logits, torch.float32, (T, E), "router_logits")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    r = routing_struct(E, renormalize, scoring, num_expert_group, topk_group, e_score_correction_bias,
                       routed_scaling_factor)
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_w8a16_workspace_bytes_ex(T, H, I, E, k, block_m, num_shared_experts,
                                                        apply_router_weight_on_input), "workspace")
    _check(lib().moe_w8a16_apply_ex(_ptr(x), act, T, H, I, E, k, _ptr(router_logits), ctypes.byref(r), _ptr(w13),
                                    _ptr(w13_scale), ld13, _ptr(w2), _ptr(w2_scale), ld2, ctypes.byref(o),
                                    _ptr(topk_w), _ptr(topk_ids), block_m, _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_w8a16_apply_ex")


def _w4_checked(x, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales, w2_qzeros, group_size, S):
    T, H, act = _need_act(x)
    Et, N2, _ = w13_qweight.shape
    I = N2 // 2
    if S < 0 or S >= Et:
        raise ValueError(f"num_shared_experts {S} must be in [0, {Et})")
    _need(w13_qweight, torch.int32, (Et, 2 * I, H // 8), "w13_qweight")
    _need(w13_scales, torch.float16, (Et, 2 * I, H // group_size), "w13_scales")
    _need(w13_qzeros, torch.int32, (Et, 2 * I // 8, H // group_size), "w13_qzeros")
    _need(w2_qweight, torch.int32, (Et, H, I // 8), "w2_qweight")
    _need(w2_scales, torch.float16, (Et, H, I // group_size), "w2_scales")
    _need(w2_qzeros, torch.int32, (Et, H // 8, I // group_size), "w2_qzeros")
    return T, H, I, Et - S, act


def moe_w4a16_forward_ex(x, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales, w2_qzeros, group_size,
                         topk_w, topk_ids, out, workspace, num_shared_experts=0, apply_router_weight_on_input=False,
                         block_m: int = 0, stream=None):
    T, H, I, E, act = _w4_checked(x, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales, w2_qzeros,
                                  group_size, num_shared_experts)
    k = topk_ids.shape[1]
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_w4a16_workspace_bytes_ex(T, H, I, E, k, block_m, num_shared_experts,
                                                        apply_router_weight_on_input), "workspace")
    _check(lib().moe_w4a16_forward_ex(_ptr(x), act, T, H, I, E, k, _ptr(w13_qweight), _ptr(w13_scales),
                                      _ptr(w13_qzeros), _ptr(w2_qweight), _ptr(w2_scales), _ptr(w2_qzeros),
                                      group_size, _ptr(topk_w), _ptr(topk_ids), ctypes.byref(o), block_m, _ptr(out),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)), "moe_w4a16_forward_ex")


def moe_w4a16_apply_ex(x, router_logits, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales, w2_qzeros,
                       group_size, topk_w, topk_ids, out, workspace, renormalize=True, scoring="softmax",
                       num_expert_group=0, topk_group=0, e_score_correction_bias=None, routed_scaling_factor=1.0,
                       num_shared_experts=0, apply_router_weight_on_input=False, block_m: int = 0, stream=None):
    T, H, I, E, act = _w4_checked(x, w13_qweight, w13_scales, w13_qzeros, w2_qweight, w2_scales, w2_qzeros,
                                  group_size, num_shared_experts)
    k = topk_ids.shape[1]
    _need(router_logits, torch.float32, (T, E), "router_logits")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    r = routing_struct(E, renormalize, scoring, num_expert_group, topk_group, e_score_correction_bias,
                       routed_scaling_factor)
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_w4a16_workspace_bytes_ex(T, H, I, E, k, block_m, num_shared_experts,
                                                        apply_router_weight_on_input), "workspace")
    _check(lib().moe_w4a16_apply_ex(_ptr(x), act, T, H, I, E, k, _ptr(router_logits), ctypes.byref(r),
                                    _ptr(w13_qweight), _ptr(w13_scales), _ptr(w13_qzeros), _ptr(w2_qweight),
                                    _ptr(w2_scales), _ptr(w2_qzeros), group_size, ctypes.byref(o), _ptr(topk_w),
                                    _ptr(topk_ids), block_m, _ptr(out), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_w4a16_apply_ex")


# ---------------------------------------------------------------------------
# GPTQ / AWQ 4-bit checkpoint import
# ---------------------------------------------------------------------------

MOE_W4_FORMAT = {"awq": 0, "gptq": 1}


def moe_wna16_group_size(H: int, I: int, group_size: int):
    """(group size, repeat) that MoeWNA16Method.create_weights settles on for a checkpoint group size."""
    g, r = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().moe_wna16_group_size(H, I, group_size, ctypes.byref(g), ctypes.byref(r)), "moe_wna16_group_size")
    return g.value, r.value


def moe_w4_import(fmt: str, qweight, qzeros, scales, N: int, K: int, group_size: int, repeat: int, out_qweight,
                  out_scales, out_qzeros, stream=None):
    """One [N, K] matrix of a 4-bit AWQ or GPTQ checkpoint into this library's layout (see moe_wq.h)."""
    if fmt not in MOE_W4_FORMAT:
        raise ValueError(f"format must be one of {sorted(MOE_W4_FORMAT)}, got {fmt!r}")
    gin = -(-K // group_size)
    gout = K * repeat // group_size
    _need(qweight, torch.int32, (K, N // 8) if fmt == "awq" else (K // 8, N), "qweight")
    _need(qzeros, torch.int32, (gin, N // 8), "qzeros")
    _need(scales, torch.float16, (gin, N), "scales")
    _need(out_qweight, torch.int32, (N, K // 8), "out_qweight")
    _need(out_scales, torch.float16, (N, gout), "out_scales")
    _need(out_qzeros, torch.int32, (N // 8, gout), "out_qzeros")
    _check(lib().moe_w4_import(MOE_W4_FORMAT[fmt], _ptr(qweight), _ptr(qzeros), _ptr(scales), N, K, group_size,
                               repeat, _ptr(out_qweight), _ptr(out_scales), _ptr(out_qzeros), _stream(stream)),
           "moe_w4_import")


# ---------------------------------------------------------------------------
# Weight-only fp8 (e4m3fn) experts
# ---------------------------------------------------------------------------


def moe_quantize_weights_fp8(w, q, scale, stream=None):
    """Per-tensor e4m3fn quantization of w [E, N, K] fp32 into q uint8 [E, N, K] and scale fp32 [E]."""
    E, N, K = w.shape
    _need(w, torch.float32, (E, N, K), "w")
    _need(q, torch.uint8, (E, N, K), "q")
    _need(scale, torch.float32, (E,), "scale")
    _check(lib().moe_quantize_weights_fp8(_ptr(w), E, N, K, _ptr(q), _ptr(scale), _stream(stream)),
           "moe_quantize_weights_fp8")


def moe_fp8_merge_w13_scales(w13, w13_shard_scales, w13_scale, stream=None):
    """w13 uint8 [E, 2I, H] with shard scales [E, 2] -> requantized in place under w13_scale [E] = the maxima."""
    E, N2, H = w13.shape
    _need(w13, torch.uint8, (E, N2, H), "w13")
    _need(w13_shard_scales, torch.float32, (E, 2), "w13_shard_scales")
    _need(w13_scale, torch.float32, (E,), "w13_scale")
    _check(lib().moe_fp8_merge_w13_scales(_ptr(w13), _ptr(w13_shard_scales), E, N2 // 2, H, _ptr(w13_scale),
                                          _stream(stream)), "moe_fp8_merge_w13_scales")


def moe_wfp8a16_workspace_bytes(T, H, I, E, k, block_m=0, num_shared_experts=0,
                                apply_router_weight_on_input=False) -> int:
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    return int(lib().moe_wfp8a16_workspace_bytes(T, H, I, E, k, block_m, ctypes.byref(o)))


def _fp8_checked(x, w13, w13_scale, w2, w2_scale, S):
    T, H, act = _need_act(x)
    Et, N2, _ = w13.shape
    I = N2 // 2
    if S < 0 or S >= Et:
        raise ValueError(f"num_shared_experts {S} must be in [0, {Et})")
    ld13 = _row_stride(w13, torch.uint8, (Et, 2 * I, H), "w13")
    _need(w13_scale, torch.float32, (Et,), "w13_scale")
    ld2 = _row_stride(w2, torch.uint8, (Et, H, I), "w2")
    _need(w2_scale, torch.float32, (Et,), "w2_scale")
    return T, H, I, Et - S, act, ld13, ld2


def moe_wfp8a16_forward(x, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, workspace, num_shared_experts=0,
                        apply_router_weight_on_input=False, block_m: int = 0, stream=None):
    T, H, I, E, act, ld13, ld2 = _fp8_checked(x, w13, w13_scale, w2, w2_scale, num_shared_experts)
    k = topk_ids.shape[1]
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_wfp8a16_workspace_bytes(T, H, I, E, k, block_m, num_shared_experts,
                                                       apply_router_weight_on_input), "workspace")
    _check(lib().moe_wfp8a16_forward(_ptr(x), act, T, H, I, E, k, _ptr(w13), _ptr(w13_scale), ld13, _ptr(w2),
                                     _ptr(w2_scale), ld2, _ptr(topk_w), _ptr(topk_ids), ctypes.byref(o), block_m, _ptr(out),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "moe_wfp8a16_forward")


def moe_wfp8a16_apply(x, router_logits, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, workspace,
                      renormalize=True, scoring="softmax", num_expert_group=0, topk_group=0,
                      e_score_correction_bias=None, routed_scaling_factor=1.0, num_shared_experts=0,
                      apply_router_weight_on_input=False, block_m: int = 0, stream=None):
    T, H, I, E, act, ld13, ld2 = _fp8_checked(x, w13, w13_scale, w2, w2_scale, num_shared_experts)
    k = topk_ids.shape[1]
    _need(router_logits, torch.float32, (T, E), "router_logits")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    r = routing_struct(E, renormalize, scoring, num_expert_group, topk_group, e_score_correction_bias,
                       routed_scaling_factor)
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_wfp8a16_workspace_bytes(T, H, I, E, k, block_m, num_shared_experts,
                                                       apply_router_weight_on_input), "workspace")
    _check(lib().moe_wfp8a16_apply(_ptr(x), act, T, H, I, E, k, _ptr(router_logits), ctypes.byref(r), _ptr(w13),
                                   _ptr(w13_scale), ld13, _ptr(w2), _ptr(w2_scale), ld2, ctypes.byref(o), _ptr(topk_w),
                                   _ptr(topk_ids), block_m, _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)), "moe_wfp8a16_apply")


# ---------------------------------------------------------------------------
# W8A8: int8 weights, int8 activations quantized per token
# ---------------------------------------------------------------------------


def moe_quantize_act_int8(x, q, scale, stream=None):
    """Per-token int8 codes q int8 [T, H] and scales fp32 [T] of the bf16/fp16 activations x [T, H]."""
    T, H, act = _need_act(x)
    _need(q, torch.int8, (T, H), "q")
    _need(scale, torch.float32, (T,), "scale")
    _check(lib().moe_quantize_act_int8(_ptr(x), act, T, H, _ptr(q), _ptr(scale), _stream(stream)),
           "moe_quantize_act_int8")


def moe_w8a8_workspace_bytes(T, H, I, E, k, block_m=0, num_shared_experts=0, apply_router_weight_on_input=False):
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    return int(lib().moe_w8a8_workspace_bytes(T, H, I, E, k, block_m, ctypes.byref(o)))


def moe_w8a8_forward(x, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, workspace, num_shared_experts=0,
                     apply_router_weight_on_input=False, block_m: int = 0, stream=None):
    T, H, I, E, act, ld13, ld2 = _w8_checked(x, w13, w13_scale, w2, w2_scale, num_shared_experts)
    k = topk_ids.shape[1]
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_w8a8_workspace_bytes(T, H, I, E, k, block_m, num_shared_experts,
                                                    apply_router_weight_on_input), "workspace")
    _check(lib().moe_w8a8_forward(_ptr(x), act, T, H, I, E, k, _ptr(w13), _ptr(w13_scale), ld13, _ptr(w2),
                                  _ptr(w2_scale), ld2, _ptr(topk_w), _ptr(topk_ids), ctypes.byref(o), block_m,
                                  _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _stream(stream)), "moe_w8a8_forward")


def moe_w8a8_apply(x, router_logits, w13, w13_scale, w2, w2_scale, topk_w, topk_ids, out, workspace,
                   renormalize=True, scoring="softmax", num_expert_group=0, topk_group=0, e_score_correction_bias=None,
                   routed_scaling_factor=1.0, num_shared_experts=0, apply_router_weight_on_input=False,
                   block_m: int = 0, stream=None):
    T, H, I, E, act, ld13, ld2 = _w8_checked(x, w13, w13_scale, w2, w2_scale, num_shared_experts)
    k = topk_ids.shape[1]
    _need(router_logits, torch.float32, (T, E), "router_logits")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(out, x.dtype, (T, H), "out")
    r = routing_struct(E, renormalize, scoring, num_expert_group, topk_group, e_score_correction_bias,
                       routed_scaling_factor)
    o = fused_opts(num_shared_experts, apply_router_weight_on_input)
    _need_bytes(workspace, moe_w8a8_workspace_bytes(T, H, I, E, k, block_m, num_shared_experts,
                                                    apply_router_weight_on_input), "workspace")
    _check(lib().moe_w8a8_apply(_ptr(x), act, T, H, I, E, k, _ptr(router_logits), ctypes.byref(r), _ptr(w13),
                                _ptr(w13_scale), ld13, _ptr(w2), _ptr(w2_scale), ld2, ctypes.byref(o), _ptr(topk_w),
                                _ptr(topk_ids), block_m, _ptr(out), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)), "moe_w8a8_apply")
