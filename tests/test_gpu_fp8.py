"""GPU weight-only fp8 experts (fp8 page, Fp8MoEMethod) against the oracle: e4m3fn codes and
per-tensor scales bit for bit (quantizer and w13 scale merge), the layer within tolerance."""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import DEV, act_f64, assert_layer_close, log, route_both, to_dev_act

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    pkg.lib()


def _gpu_quant(w):
    E = w.shape[0]
    q = torch.empty(w.shape, dtype=torch.uint8, device=DEV)
    s = torch.empty(E, dtype=torch.float32, device=DEV)
    pkg.moe_quantize_weights_fp8(torch.from_numpy(np.ascontiguousarray(w)).to(DEV), q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def test_quantizer_ties_and_signs():
    """Max 448 gives scale 1, so w / scale = w and every rounding case of e4m3 is exercised."""
    v = np.array([448.0, 1.0625, 1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -2.0 ** -10, 0.0, -0.0, 44.8, -447.0,
                  0.0155, 2.0 ** -6, 15.5, 17.0, 300.0, -1e-5], np.float32)
    w = np.tile(v, 8).reshape(1, 8, 16)
    q, s = _gpu_quant(w)
    qr, sr = oracle.quantize_fp8_tensor(w[0])
    assert s[0] == sr == 1.0
    np.testing.assert_array_equal(q[0], qr)


@pytest.mark.parametrize("E,N,K,scale", [(3, 64, 256, 0.02), (2, 300, 130, 1e-3), (1, 8, 8, 0.0)])
def test_quantizer_bit_exact(E, N, K, scale):
    w = (synthetic.random_master((E, N, K), E * N + K, tag=90) * np.float32(scale / 0.02)).astype(np.float32)
    w[0, 0, :4] = [-0.0, 0.0, w[0, 0, 4], -w[0, 0, 4]]
    q, s = _gpu_quant(w)
    for e in range(E):
        qr, sr = oracle.quantize_fp8_tensor(w[e])
        assert s[e].view(np.uint32) == np.float32(sr).view(np.uint32)
        np.testing.assert_array_equal(q[e], qr)


def test_w13_merge_bit_exact():
    E, I, H = 4, 96, 128
    w = synthetic.random_master((E, 2 * I, H), 11, tag=91)
    q13 = np.empty((E, 2 * I, H), np.uint8)
    s13 = np.empty((E, 2), np.float32)
    for e in range(E):
        for sh in range(2):
            part = w[e, sh * I:(sh + 1) * I] * np.float32(1.0 + 0.7 * sh * (e % 2))
            q13[e, sh * I:(sh + 1) * I], s13[e, sh] = oracle.quantize_fp8_tensor(part)
    dq = torch.from_numpy(q13).to(DEV)
    out_s = torch.empty(E, dtype=torch.float32, device=DEV)
    pkg.moe_fp8_merge_w13_scales(dq, torch.from_numpy(s13).to(DEV), out_s)
    torch.cuda.synchronize()
    qr, sr = oracle.fp8_merge_w13_scales(q13, s13)
    np.testing.assert_array_equal(out_s.cpu().numpy(), sr)
    np.testing.assert_array_equal(dq.cpu().numpy(), qr)


class FP8Weights:
    def __init__(self, E, H, I, seed):
        self.E, self.H, self.I = E, H, I
        self.layer = pkg.WFP8A16MoE(E, H, I, device=DEV)
        self.q13 = np.empty((E, 2 * I, H), np.uint8)
        self.q2 = np.empty((E, H, I), np.uint8)
        self.s13 = np.empty(E, np.float32)
        self.s2 = np.empty(E, np.float32)
        for e in range(E):
            m13 = synthetic.random_master((2 * I, H), seed * 100 + e, tag=92)
            m2 = synthetic.random_master((H, I), seed * 100 + e, tag=93)
            self.layer.load_expert(e, torch.from_numpy(m13).to(DEV), torch.from_numpy(m2).to(DEV))
            self.q13[e], self.s13[e] = oracle.quantize_fp8_tensor(m13)
            self.q2[e], self.s2[e] = oracle.quantize_fp8_tensor(m2)
        torch.cuda.synchronize()
        assert np.array_equal(self.layer.w13_weight.cpu().numpy(), self.q13)
        assert np.array_equal(self.layer.w2_weight_scale.cpu().numpy(), self.s2)


@pytest.mark.parametrize("act,T,bm", [("bf16", 5, 0), ("fp16", 61, 32), ("bf16", 130, 64), ("bf16", 700, 256),
                                      ("fp16", 37, 0), ("bf16", 1, 16)])
def test_layer(act, T, bm):
    E, k, H, I = 8, 2, 512, 1024
    log(f"[fp8] act={act} T={T} block_m={bm}")
    W = FP8Weights(E, H, I, seed=3)
    xb = synthetic.random_activations(T, H, act, seed=T)
    logits = synthetic.random_logits(T, E, seed=T + 1)
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    x = to_dev_act(xb, act)
    out = W.layer.forward_topk(x, tw, ti, block_m=bm)
    torch.cuda.synchronize()
    ref = oracle.moe_forward_fp8(act_f64(xb, act), W.q13, W.s13, W.q2, W.s2, w_ref, ids_ref)
    assert_layer_close(out.float().cpu().numpy().astype(np.float64), ref, f"fp8 {act} T={T} bm={bm}")


@pytest.mark.parametrize("T,bm", [(3, 16), (40, 32)])
def test_layer_odd_shapes(T, bm):
    """The 16/32-row streaming GEMMs with H = 3 x 128 (three column tiles) and I = 10 x 64 (K parts of
    uneven length)."""
    E, k, H, I = 8, 2, 384, 640
    log(f"[fp8] odd shapes T={T} block_m={bm}")
    W = FP8Weights(E, H, I, seed=6)
    xb = synthetic.random_activations(T, H, "bf16", seed=T + 3)
    logits = synthetic.random_logits(T, E, seed=T + 4)
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    out = W.layer.forward_topk(to_dev_act(xb, "bf16"), tw, ti, block_m=bm)
    torch.cuda.synchronize()
    ref = oracle.moe_forward_fp8(act_f64(xb, "bf16"), W.q13, W.s13, W.q2, W.s2, w_ref, ids_ref)
    assert_layer_close(out.float().cpu().numpy().astype(np.float64), ref, f"fp8 odd shapes T={T} bm={bm}")


def test_layer_apply_with_options():
    """Routing from logits with grouped sigmoid routing, a shared expert and the weight on the input."""
    E, k, H, I, T, S = 8, 2, 256, 512, 45, 1
    W = FP8Weights(E + S, H, I, seed=4)
    xb = synthetic.random_activations(T, H, "bf16", seed=5)
    logits = synthetic.random_logits(T, E, seed=6)
    bias = (0.1 * np.random.default_rng(7).standard_normal(E)).astype(np.float32)
    x = to_dev_act(xb, "bf16")
    out = torch.empty_like(x)
    tw = torch.empty(T, k, dtype=torch.float32, device=DEV)
    ti = torch.empty(T, k, dtype=torch.int32, device=DEV)
    ws = torch.empty(pkg.moe_wfp8a16_workspace_bytes(T, H, I, E, k, 0, S, True), dtype=torch.uint8, device=DEV)
    L = W.layer
    pkg.moe_wfp8a16_apply(x, torch.from_numpy(logits).to(DEV), L.w13_weight, L.w13_weight_scale, L.w2_weight,
                          L.w2_weight_scale, tw, ti, out, ws, scoring="sigmoid", num_expert_group=4, topk_group=2,
                          e_score_correction_bias=torch.from_numpy(bias).to(DEV), routed_scaling_factor=2.0,
                          num_shared_experts=S, apply_router_weight_on_input=True)
    torch.cuda.synchronize()
    w_ref, ids_ref = oracle.route_select(logits, k, True, "sigmoid", 4, 2, bias, 2.0)
    np.testing.assert_array_equal(ti.cpu().numpy(), ids_ref)
    ref = oracle.moe_forward_fp8(act_f64(xb, "bf16"), W.q13, W.s13, W.q2, W.s2, w_ref, ids_ref,
                                 weight_on_input=True, num_shared=S)
    assert_layer_close(out.float().cpu().numpy().astype(np.float64), ref, "fp8 apply with options")


_MIXTRAL_FP8 = {}


def _mixtral_fp8_weights():
    if not _MIXTRAL_FP8:
        _MIXTRAL_FP8["w"] = FP8Weights(8, 4096, 14336, seed=5)
    return _MIXTRAL_FP8["w"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [1, 64])
def test_mixtral_decode_fp8(T):
    """Mixtral-sized experts at decode size (blocks of 16 and 32 rows: the streaming GEMM1 with e4m3
    decoding and the streaming fp8 GEMM2, K cut into several parts); every row against the oracle."""
    E, k, H, I = 8, 2, 4096, 14336
    assert pkg.moe_w8a16_block_m(T, H, I, E, k) in (16, 32)
    log(f"[fp8] mixtral decode T={T}")
    W = _mixtral_fp8_weights()
    xb = synthetic.random_activations(T, H, "bf16", seed=9 + T)
    logits = synthetic.random_logits(T, E, seed=10 + T)
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    out = W.layer.forward_topk(to_dev_act(xb, "bf16"), tw, ti)
    again = W.layer.forward_topk(to_dev_act(xb, "bf16"), tw, ti)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "two runs differ bitwise"
    ref = oracle.moe_forward_fp8(act_f64(xb, "bf16"), W.q13, W.s13, W.q2, W.s2, w_ref, ids_ref)
    assert_layer_close(out.float().cpu().numpy().astype(np.float64), ref, f"fp8 mixtral decode T={T}")


@pytest.mark.timeout(900)
def test_mixtral_prefill_fp8_sampled():
    """Mixtral-sized experts at prefill size (256-row blocks: the 256-row GEMM1 with e4m3 decoding and the
    planes GEMM2): each output row depends only on its own token, so the oracle checks 8 sampled rows."""
    E, k, H, I, T = 8, 2, 4096, 14336, 1024
    assert pkg.moe_w8a16_block_m(T, H, I, E, k) == 256
    log(f"[fp8] mixtral prefill T={T}")
    W = _mixtral_fp8_weights()
    xb = synthetic.random_activations(T, H, "bf16", seed=7)
    logits = synthetic.random_logits(T, E, seed=8)
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    out = W.layer.forward_topk(to_dev_act(xb, "bf16"), tw, ti)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, T - 1, 8).astype(int))
    ref = oracle.moe_forward_fp8(act_f64(xb[rows], "bf16"), W.q13, W.s13, W.q2, W.s2, w_ref[rows], ids_ref[rows])
    got = out.float().cpu().numpy().astype(np.float64)[rows]
    assert_layer_close(got, ref, f"fp8 mixtral prefill T={T} sampled rows")
