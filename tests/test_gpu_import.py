"""GPU import of 4-bit AWQ and GPTQ checkpoint tensors (moe_wna16 page, get_weight_loader) against
the oracle's import, bit for bit, and a layer run on imported weights against the oracle layer."""
import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import DEV, act_f64, assert_layer_close, log, to_dev_act
from test_oracle_import import pack_awq_qweight, pack_awq_qzeros, pack_gptq_qweight, pack_gptq_qzeros

pytestmark = pytest.mark.gpu


def _checkpoint(fmt, N, Kfull, K, g, seed):
    """A synthetic checkpoint matrix: codes, fp16 scales and zeros of g-wide groups over Kfull columns,
    cut to K columns (the last group partial when g does not divide K), packed as `fmt` stores it."""
    w = synthetic.random_master((N, Kfull), seed, tag=82)
    q, s, z = oracle.quantize_w4_groups(w, g)
    gin = -(-K // g)
    q, s, z = q[:, :K], s[:, :gin], np.maximum(z[:, :gin], 1 if fmt == "gptq" else 0).astype(np.uint8)
    if fmt == "awq":
        return pack_awq_qweight(q), pack_awq_qzeros(z), np.ascontiguousarray(s.T)
    return pack_gptq_qweight(q), pack_gptq_qzeros(z), np.ascontiguousarray(s.T)


def _gpu_import(fmt, qw, qz, sc, N, K, g, repeat):
    gout = K * repeat // g
    oq = torch.empty(N, K // 8, dtype=torch.int32, device=DEV)
    osc = torch.empty(N, gout, dtype=torch.float16, device=DEV)
    oz = torch.empty(N // 8, gout, dtype=torch.int32, device=DEV)
    pkg.moe_w4_import(fmt, torch.from_numpy(qw).to(DEV), torch.from_numpy(qz).to(DEV),
                      torch.from_numpy(sc).to(DEV), N, K, g, repeat, oq, osc, oz)
    torch.cuda.synchronize()
    return oq.cpu().numpy(), osc.cpu().numpy(), oz.cpu().numpy()


@pytest.mark.parametrize("fmt", ["awq", "gptq"])
@pytest.mark.parametrize("N,K,H,I,g", [(64, 256, 256, 256, 128), (2048, 1408, 2048, 1408, 256),
                                      (1408, 2048, 2048, 1408, 256), (48, 512, 512, 512, 64)])
def test_import_bit_exact(fmt, N, K, H, I, g):
    g2, rep = pkg.moe_wna16_group_size(H, I, g)
    assert (g2, rep) == oracle.wna16_group_size(H, I, g)
    log(f"[import] {fmt} N={N} K={K} g={g} -> {g2} x{rep}")
    qw, qz, sc = _checkpoint(fmt, N, -(-K // g) * g, K, g, seed=N + K)
    got = _gpu_import(fmt, qw, qz, sc, N, K, g, rep)
    ref = (oracle.import_awq if fmt == "awq" else oracle.import_gptq)(qw, qz, sc, H=H, I=I, group_size=g)
    gout = K // g2
    np.testing.assert_array_equal(got[0], ref[0])
    np.testing.assert_array_equal(got[1].view(np.uint16), ref[1][:, :gout].view(np.uint16))
    np.testing.assert_array_equal(got[2], ref[2][:, :gout])


def test_gptq_stored_fifteen_carries_like_the_page():
    N, K, g = 16, 128, 128
    qw = np.zeros((K // 8, N), np.int32)
    qz = np.array([[0x0000003F, 0x7FFFFFFF]], np.uint32).view(np.int32)
    sc = np.ones((1, N), np.float16)
    got = _gpu_import("gptq", qw, qz, sc, N, K, g, 1)
    ref = oracle.import_gptq(qw, qz, sc, H=K, I=K, group_size=g)
    np.testing.assert_array_equal(got[2], ref[2])


@pytest.mark.parametrize("fmt", ["awq", "gptq"])
def test_layer_on_imported_weights(fmt):
    """A whole W4A16 layer loaded from an AWQ / GPTQ checkpoint (g = 256 halved to 128 for I = 640)."""
    E, k, H, I, g, T = 4, 2, 512, 640, 256, 19
    g2, rep = pkg.moe_wna16_group_size(H, I, g)
    assert (g2, rep) == (128, 2)
    qw13 = torch.empty(E, 2 * I, H // 8, dtype=torch.int32, device=DEV)
    sc13 = torch.empty(E, 2 * I, H // g2, dtype=torch.float16, device=DEV)
    qz13 = torch.empty(E, 2 * I // 8, H // g2, dtype=torch.int32, device=DEV)
    qw2 = torch.empty(E, H, I // 8, dtype=torch.int32, device=DEV)
    sc2 = torch.empty(E, H, I // g2, dtype=torch.float16, device=DEV)
    qz2 = torch.empty(E, H // 8, I // g2, dtype=torch.int32, device=DEV)
    host = {key: [] for key in ("qw13", "sc13", "qz13", "qw2", "sc2", "qz2")}
    imp = oracle.import_awq if fmt == "awq" else oracle.import_gptq
    for e in range(E):
        parts = []
        for half in range(2):         # gate rows, then up rows
            qw, qz, sc = _checkpoint(fmt, I, -(-H // g) * g, H, g, seed=100 * e + half)
            rows = slice(half * I, (half + 1) * I)
            zrows = slice(half * I // 8, (half + 1) * I // 8)
            pkg.moe_w4_import(fmt, torch.from_numpy(qw).to(DEV), torch.from_numpy(qz).to(DEV),
                              torch.from_numpy(sc).to(DEV), I, H, g, rep, qw13[e, rows], sc13[e, rows],
                              qz13[e, zrows])
            parts.append(imp(qw, qz, sc, H=H, I=I, group_size=g))
        host["qw13"].append(np.concatenate([p[0] for p in parts]))
        host["sc13"].append(np.concatenate([p[1][:, :H // g2] for p in parts]))
        host["qz13"].append(np.concatenate([p[2][:, :H // g2] for p in parts]))
        qw, qz, sc = _checkpoint(fmt, H, -(-I // g) * g, I, g, seed=100 * e + 7)
        pkg.moe_w4_import(fmt, torch.from_numpy(qw).to(DEV), torch.from_numpy(qz).to(DEV),
                          torch.from_numpy(sc).to(DEV), H, I, g, rep, qw2[e], sc2[e], qz2[e])
        p2 = imp(qw, qz, sc, H=H, I=I, group_size=g)
        host["qw2"].append(p2[0]); host["sc2"].append(p2[1][:, :I // g2]); host["qz2"].append(p2[2][:, :I // g2])
    torch.cuda.synchronize()
    h = {key: np.stack(v) for key, v in host.items()}
    np.testing.assert_array_equal(qw13.cpu().numpy(), h["qw13"])
    np.testing.assert_array_equal(qz2.cpu().numpy(), h["qz2"])
    xb = synthetic.random_activations(T, H, "fp16", seed=3)
    w_ref, ids_ref = oracle.route_softmax_topk(synthetic.random_logits(T, E, seed=4), k, True)
    x = to_dev_act(xb, "fp16")
    out = torch.empty_like(x)
    ws = torch.empty(pkg.moe_w4a16_workspace_bytes(T, H, I, E, k, 0), dtype=torch.uint8, device=DEV)
    pkg.moe_w4a16_forward(x, qw13, sc13, qz13, qw2, sc2, qz2, g2, torch.from_numpy(w_ref.astype(np.float32)).to(DEV),
                          torch.from_numpy(ids_ref).to(DEV), out, ws)
    torch.cuda.synchronize()
    ref = oracle.moe_forward_w4(act_f64(xb, "fp16"), h["qw13"], h["sc13"], h["qz13"], h["qw2"], h["sc2"], h["qz2"],
                                g2, w_ref.astype(np.float32).astype(np.float64), ids_ref)
    assert_layer_close(out.float().cpu().numpy().astype(np.float64), ref, f"layer on {fmt} weights")
