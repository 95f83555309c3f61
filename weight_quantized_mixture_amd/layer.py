"""Layer objects holding quantized expert parameters in device memory.

Parameter names and shapes follow the pages:
  experts_int8 page, ExpertsInt8MoEMethod.create_weights:
    w13_weight int8 [E, 2I, H] (gate rows then up rows), w2_weight int8 [E, H, I],
    w13_scale fp32 [E, 2I], w2_scale fp32 [E, H];
  moe_wna16 page, MoeWNA16Method.create_weights (4-bit, packed 8 per int32 here):
    w13_qweight [E, 2I, H/8], w2_qweight [E, H, I/8], w13_scales fp16 [E, 2I, H/g],
    w2_scales fp16 [E, H, I/g], w13_qzeros [E, 2I/8, H/g], w2_qzeros [E, H/8, I/g].
``apply`` routes (moe_route_topk) and runs the fused forward on the current
stream; ``forward_topk`` takes precomputed routing like the moe_wna16 page's
``apply``.  torch only provides the device buffers.
"""
from __future__ import annotations

import torch

from . import binding as B


def padded_rows(E: int, N: int, K: int, dtype, device) -> torch.Tensor:
    """[E, N, K] view whose rows are padded by 256 bytes when a row is a multiple of 512 bytes.

    Rows that start a multiple of 512 bytes apart fall on the same HBM channels when a wave
    reads 16 of them at the same offset; the fp8 page pads such rows on ROCm for the same
    reason (Fp8LinearMethod._maybe_pad_weight).  The library reads the row stride.
    """
    itemsize = torch.empty(0, dtype=dtype).element_size()
    row_bytes = K * itemsize
    ld = K + 256 // itemsize if row_bytes % 512 == 0 else K
    return torch.empty(E, N, ld, dtype=dtype, device=device)[:, :, :K]


class _Workspace:
    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


class W8A16MoE:
    def __init__(self, num_experts: int, hidden_size: int, intermediate_size: int,
                 device="cuda", params_dtype=torch.bfloat16):
        E, H, I = num_experts, hidden_size, intermediate_size
        self.E, self.H, self.I = E, H, I
        self.params_dtype = params_dtype
        self.w13_weight = padded_rows(E, 2 * I, H, torch.int8, device)
        self.w2_weight = padded_rows(E, H, I, torch.int8, device)
        self.w13_scale = torch.zeros(E, 2 * I, dtype=torch.float32, device=device)
        self.w2_scale = torch.zeros(E, H, dtype=torch.float32, device=device)
        self._ws = _Workspace()

    def load_expert(self, e: int, w13_master: torch.Tensor, w2_master: torch.Tensor):
        """Quantize one expert's fp32 masters ([2I, H] gate then up, [H, I]) into the int8 parameters."""
        q = torch.empty(1, 2 * self.I, self.H, dtype=torch.int8, device=w13_master.device)
        B.moe_quantize_weights_int8(w13_master.reshape(1, 2 * self.I, self.H), q, self.w13_scale[e:e + 1])
        self.w13_weight[e].copy_(q[0])
        q = torch.empty(1, self.H, self.I, dtype=torch.int8, device=w2_master.device)
        B.moe_quantize_weights_int8(w2_master.reshape(1, self.H, self.I), q, self.w2_scale[e:e + 1])
        self.w2_weight[e].copy_(q[0])

    def route(self, router_logits: torch.Tensor, top_k: int, renormalize: bool = True):
        T = router_logits.shape[0]
        topk_w = torch.empty(T, top_k, dtype=torch.float32, device=router_logits.device)
        topk_ids = torch.empty(T, top_k, dtype=torch.int32, device=router_logits.device)
        B.moe_route_topk(router_logits, top_k, renormalize, topk_w, topk_ids)
        return topk_w, topk_ids

    def forward_topk(self, x, topk_w, topk_ids, out=None, block_m: int = 0):
        T = x.shape[0]
        k = topk_ids.shape[1]
        if out is None:
            out = torch.empty_like(x)
        ws = self._ws.get(B.moe_w8a16_workspace_bytes(T, self.H, self.I, self.E, k, block_m), x.device)
        B.moe_w8a16_forward(x, self.w13_weight, self.w13_scale, self.w2_weight, self.w2_scale, topk_w,
                            topk_ids, out, ws, block_m)
        return out

    def apply(self, x, router_logits, top_k: int, renormalize: bool = True, inplace: bool = False,
              block_m: int = 0):
        """Route from logits and run the layer (one library call); returns the output."""
        T = x.shape[0]
        out = x if inplace else torch.empty_like(x)
        self.topk_w = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
        self.topk_ids = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
        ws = self._ws.get(B.moe_w8a16_workspace_bytes(T, self.H, self.I, self.E, top_k, block_m), x.device)
        B.moe_w8a16_apply(x, router_logits, renormalize, self.w13_weight, self.w13_scale, self.w2_weight,
                          self.w2_scale, self.topk_w, self.topk_ids, out, ws, block_m)
        return out


class W4A16MoE:
    def __init__(self, num_experts: int, hidden_size: int, intermediate_size: int, group_size: int = 128,
                 device="cuda", params_dtype=torch.float16):
        E, H, I, g = num_experts, hidden_size, intermediate_size, group_size
        self.E, self.H, self.I, self.group_size = E, H, I, g
        self.params_dtype = params_dtype
        self.w13_qweight = torch.empty(E, 2 * I, H // 8, dtype=torch.int32, device=device)
        self.w2_qweight = torch.empty(E, H, I // 8, dtype=torch.int32, device=device)
        self.w13_scales = torch.zeros(E, 2 * I, H // g, dtype=torch.float16, device=device)
        self.w2_scales = torch.zeros(E, H, I // g, dtype=torch.float16, device=device)
        self.w13_qzeros = torch.zeros(E, 2 * I // 8, H // g, dtype=torch.int32, device=device)
        self.w2_qzeros = torch.zeros(E, H // 8, I // g, dtype=torch.int32, device=device)
        self._ws = _Workspace()

    def load_expert(self, e: int, w13_master: torch.Tensor, w2_master: torch.Tensor):
        g = self.group_size
        B.moe_quantize_weights_w4(w13_master.reshape(1, 2 * self.I, self.H), g, self.w13_qweight[e:e + 1],
                                  self.w13_scales[e:e + 1], self.w13_qzeros[e:e + 1])
        B.moe_quantize_weights_w4(w2_master.reshape(1, self.H, self.I), g, self.w2_qweight[e:e + 1],
                                  self.w2_scales[e:e + 1], self.w2_qzeros[e:e + 1])

    route = W8A16MoE.route

    def forward_topk(self, x, topk_w, topk_ids, out=None, block_m: int = 0):
        T = x.shape[0]
        k = topk_ids.shape[1]
        if out is None:
            out = torch.empty_like(x)
        ws = self._ws.get(B.moe_w4a16_workspace_bytes(T, self.H, self.I, self.E, k, block_m), x.device)
        B.moe_w4a16_forward(x, self.w13_qweight, self.w13_scales, self.w13_qzeros, self.w2_qweight,
                            self.w2_scales, self.w2_qzeros, self.group_size, topk_w, topk_ids, out, ws,
                            block_m)
        return out

    def apply(self, x, router_logits, top_k: int, renormalize: bool = True, inplace: bool = False,
              block_m: int = 0):
        T = x.shape[0]
        out = x if inplace else torch.empty_like(x)
        self.topk_w = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
        self.topk_ids = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
        ws = self._ws.get(B.moe_w4a16_workspace_bytes(T, self.H, self.I, self.E, top_k, block_m), x.device)
        B.moe_w4a16_apply(x, router_logits, renormalize, self.w13_qweight, self.w13_scales, self.w13_qzeros,
                          self.w2_qweight, self.w2_scales, self.w2_qzeros, self.group_size, self.topk_w,
                          self.topk_ids, out, ws, block_m)
        return out


class WFP8A16MoE:
    """Weight-only fp8 experts, named as on the fp8 page (Fp8MoEMethod.create_weights):
    w13_weight / w2_weight (e4m3fn codes, uint8 here), w13_weight_scale / w2_weight_scale
    (one fp32 scale per expert after process_weights_after_loading)."""

    def __init__(self, num_experts: int, hidden_size: int, intermediate_size: int, device="cuda",
                 params_dtype=torch.bfloat16):
        E, H, I = num_experts, hidden_size, intermediate_size
        self.E, self.H, self.I = E, H, I
        self.params_dtype = params_dtype
        self.w13_weight = padded_rows(E, 2 * I, H, torch.uint8, device)
        self.w2_weight = padded_rows(E, H, I, torch.uint8, device)
        self.w13_weight_scale = torch.zeros(E, dtype=torch.float32, device=device)
        self.w2_weight_scale = torch.zeros(E, dtype=torch.float32, device=device)
        self._ws = _Workspace()

    def load_expert(self, e: int, w13_master: torch.Tensor, w2_master: torch.Tensor):
        """Quantize one expert's 16/32-bit masters (scaled_fp8_quant: one scale for w13, one for w2),
        through unpadded codes copied into the (possibly row-padded) weight tensors."""
        for master, dst, scale, N, K in ((w13_master, self.w13_weight, self.w13_weight_scale, 2 * self.I, self.H),
                                         (w2_master, self.w2_weight, self.w2_weight_scale, self.H, self.I)):
            q = torch.empty(1, N, K, dtype=torch.uint8, device=dst.device)
            B.moe_quantize_weights_fp8(master.reshape(1, N, K).float().contiguous(), q, scale[e:e + 1])
            dst[e:e + 1].copy_(q)

    route = W8A16MoE.route

    def forward_topk(self, x, topk_w, topk_ids, out=None, block_m: int = 0):
        T, k = x.shape[0], topk_ids.shape[1]
        if out is None:
            out = torch.empty_like(x)
        ws = self._ws.get(B.moe_wfp8a16_workspace_bytes(T, self.H, self.I, self.E, k, block_m), x.device)
        B.moe_wfp8a16_forward(x, self.w13_weight, self.w13_weight_scale, self.w2_weight, self.w2_weight_scale,
                              topk_w, topk_ids, out, ws, block_m=block_m)
        return out

    def apply(self, x, router_logits, top_k: int, renormalize: bool = True, inplace: bool = False,
              block_m: int = 0):
        T = x.shape[0]
        out = x if inplace else torch.empty_like(x)
        self.topk_w = torch.empty(T, top_k, dtype=torch.float32, device=x.device)
        self.topk_ids = torch.empty(T, top_k, dtype=torch.int32, device=x.device)
        ws = self._ws.get(B.moe_wfp8a16_workspace_bytes(T, self.H, self.I, self.E, top_k, block_m), x.device)
        B.moe_wfp8a16_apply(x, router_logits, self.w13_weight, self.w13_weight_scale, self.w2_weight,
                            self.w2_weight_scale, self.topk_w, self.topk_ids, out, ws, renormalize=renormalize,
                            block_m=block_m)
        return out
