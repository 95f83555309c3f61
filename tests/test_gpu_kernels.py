"""GPU parity of the single kernels against the oracle: the int8 and uint4
quantizers and the align permutation bit for bit, router ids bit for bit and
weights within 1e-6, GEMM1's SiLU-gated intermediate against fp64."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import weight_quantized_mixture_amd as pkg
from weight_quantized_mixture_amd import synthetic

from moe_cases import DEV, log, route_both, small_w8, to_dev_act

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    pkg.lib()


def _quant_gpu(w):
    E, N, K = w.shape
    q = torch.empty(E, N, K, dtype=torch.int8, device=DEV)
    s = torch.empty(E, N, dtype=torch.float32, device=DEV)
    pkg.moe_quantize_weights_int8(torch.from_numpy(w).to(DEV), q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def test_quantize_int8_golden():
    g = json.load(open(os.path.join(GOLD, "quantize_int8_handworked.json")))
    q, s = _quant_gpu(np.array([g["w"]], np.float32))
    np.testing.assert_array_equal(q[0], np.array(g["q"], np.int8))
    np.testing.assert_array_equal(s[0], np.array(g["scale"], np.float32))


@pytest.mark.parametrize("shape", [(3, 64, 257), (2, 96, 512), (1, 5, 14336), (4, 33, 4)])
def test_quantize_int8_random(shape):
    log(f"[quantize_int8] shape={shape}")
    w = synthetic.random_master(shape, seed=sum(shape))
    w[0, 1, :] = 0.0                    # an all-zero row
    q, s = _quant_gpu(w)
    qr, sr = oracle.quantize_int8_rows(w)
    np.testing.assert_array_equal(s.view(np.uint32), sr.view(np.uint32))
    np.testing.assert_array_equal(q, qr)


def test_quantize_int8_halfway_cases():
    # rows whose quotients sit on or next to k + 1/2, where divide, reciprocal and rounding mode differ
    rng = np.random.default_rng(0)
    rows = []
    for _ in range(256):
        m = np.float32(rng.uniform(0.01, 0.1))
        s = np.float32(m / np.float32(127))
        kk = int(rng.integers(0, 126))
        w = np.float32((kk + 0.5) * float(s))
        rows.append([m, np.nextafter(w, np.float32(-1)), w, np.nextafter(w, np.float32(1))])
    w = np.array(rows, np.float32)[None]
    q, s = _quant_gpu(w)
    qr, sr = oracle.quantize_int8_rows(w)
    np.testing.assert_array_equal(q, qr)


@pytest.mark.parametrize("group", [8, 32, 128])
def test_quantize_w4_random_and_golden(group):
    g = json.load(open(os.path.join(GOLD, "w4_handworked.json")))
    w = synthetic.random_master((2, 24, 256), seed=group)
    w[0, 3, :group] = 0.0               # a flat group
    w[1, 0, :8] = np.array(g["w"], np.float32)
    qw = torch.empty(2, 24, 32, dtype=torch.int32, device=DEV)
    sc = torch.empty(2, 24, 256 // group, dtype=torch.float16, device=DEV)
    qz = torch.empty(2, 3, 256 // group, dtype=torch.int32, device=DEV)
    pkg.moe_quantize_weights_w4(torch.from_numpy(w).to(DEV), group, qw, sc, qz)
    torch.cuda.synchronize()
    q, s, z = oracle.quantize_w4_groups(w, group)
    np.testing.assert_array_equal(qw.cpu().numpy(), oracle.pack_w4_along_k(q))
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint16), s.view(np.uint16))
    np.testing.assert_array_equal(qz.cpu().numpy(), np.stack([oracle.pack_w4_along_n(z[e]) for e in range(2)]))
    if group == 8:
        assert format(int(qw.cpu().numpy().view(np.uint32)[1, 0, 0]), "08X") == g["packed_word_hex"]


@pytest.mark.parametrize("T,E,k,renorm", [(37, 8, 2, True), (16, 64, 6, True), (33, 128, 8, True),
                                          (5, 1024, 8, True), (9, 5, 5, False), (64, 8, 1, True),
                                          (3, 100, 7, False), (1, 1, 1, True), (12, 256, 16, True),
                                          (7, 257, 3, True), (4, 65, 65, True)])
def test_route(T, E, k, renorm):
    # E <= 256 takes the rank path, larger E the arg-max rounds
    log(f"[route] T={T} E={E} k={k} renorm={renorm}")
    logits = synthetic.random_logits(T, E, seed=T * E + k)
    if E >= 4:
        logits[0, 1] = logits[0, 3] = np.float32(logits[0].max() + 1)   # a tie at the top
    if E >= 8 and T >= 2:
        # -0 and +0 compare equal: the lower id wins
        logits[1] = -np.abs(logits[1]) - np.float32(1)
        logits[1, 6] = np.float32(0.0)
        logits[1, 2] = np.float32(-0.0)
    tw, ti, w_ref, ids_ref = route_both(logits, k, renorm)
    np.testing.assert_array_equal(ti.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(tw.cpu().numpy(), w_ref, rtol=0, atol=1e-6)
    if k == 1 and renorm:
        assert np.all(tw.cpu().numpy() == 1.0)


def test_route_t0():
    tw = torch.empty(0, 2, dtype=torch.float32, device=DEV)
    ti = torch.empty(0, 2, dtype=torch.int32, device=DEV)
    pkg.moe_route_topk(torch.empty(0, 8, dtype=torch.float32, device=DEV), 2, True, tw, ti)
    torch.cuda.synchronize()


def _align_gpu(ids, E, bm):
    T, k = ids.shape
    cap = pkg.moe_align_capacity(T, k, E, bm)
    s = torch.full((max(cap, 1),), -7, dtype=torch.int32, device=DEV)[:cap]
    b = torch.full((max(cap // bm, 1),), -7, dtype=torch.int32, device=DEV)[:cap // bm]
    n = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    pkg.moe_align_block(torch.from_numpy(ids).to(DEV), E, bm, s, b, n)
    torch.cuda.synchronize()
    return s.cpu().numpy(), b.cpu().numpy(), int(n.item())


@pytest.mark.parametrize("T,k,E,bm,skew", [(3, 2, 4, 2, False), (37, 6, 64, 16, True), (64, 2, 8, 32, False),
                                           (4096, 2, 8, 64, True), (512, 6, 64, 16, True), (1, 8, 128, 16, False),
                                           (256, 8, 128, 32, False), (100, 3, 1, 16, False),
                                           (300, 4, 1024, 16, False), (129, 2, 8, 1, False),
                                           (77, 3, 16, 128, True), (4096, 2, 8, 256, False),
                                           (1000, 3, 40, 16, True), (4096, 2, 96, 16, False),
                                           (171, 4, 129, 32, True)])
def test_align(T, k, E, bm, skew):
    log(f"[align] T={T} k={k} E={E} bm={bm} skew={skew}")
    rng = np.random.default_rng(T + E + bm)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if skew:
        ids[: (3 * T) // 4, 0] = 0
    s, b, n = _align_gpu(ids, E, bm)
    sr, br, nr = oracle.align_block(ids, E, bm)
    assert n == nr
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(b, br)


def test_align_drops_out_of_range_ids():
    ids = np.array([[0, 9], [-1, 1], [1, 0], [5, 5]], np.int32)
    s, b, n = _align_gpu(ids, 2, 2)
    sr, br, nr = oracle.align_block(ids, 2, 2)
    assert n == nr
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(b, br)
    # past 512 assignments (every chunk ranked at once): ids below 0 and at or past E in every chunk
    rng = np.random.default_rng(11)
    ids = rng.integers(-3, 70, size=(700, 3)).astype(np.int32)
    s, b, n = _align_gpu(ids, 64, 16)
    sr, br, nr = oracle.align_block(ids, 64, 16)
    assert n == nr
    np.testing.assert_array_equal(s, sr)
    np.testing.assert_array_equal(b, br)


def test_align_empty():
    n = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    e = torch.empty(0, dtype=torch.int32, device=DEV)
    pkg.moe_align_block(torch.empty(0, 2, dtype=torch.int32, device=DEV), 8, 16, e, e, n)
    torch.cuda.synchronize()
    assert int(n.item()) == 0


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_gemm1_q16_blocks_of_256(act):
    # 256-row blocks with H a multiple of 256: GEMM1 writes the 16-bit
    # fixed-point form itself, at the start of the intermediate
    E, k, H, I, T, bm = 4, 2, 512, 384, 300, 256
    log(f"[gemm1 q16] act={act} E={E} H={H} I={I} T={T}")
    W = small_w8(E, H, I, seed=13)
    xb = synthetic.random_activations(T, H, act, seed=14)
    logits = synthetic.random_logits(T, E, seed=15)
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    cap = pkg.moe_align_capacity(T, k, E, bm)
    s = torch.empty(cap, dtype=torch.int32, device=DEV)
    b = torch.empty(cap // bm, dtype=torch.int32, device=DEV)
    n = torch.empty(1, dtype=torch.int32, device=DEV)
    pkg.moe_align_block(ti, E, bm, s, b, n)
    nbytes = pkg.moe_w8a16_intermediate_bytes(T, H, I, E, k, bm)
    a = torch.full(((nbytes + 1) // 2,), 0x7FC0, dtype=torch.int16, device=DEV)
    pkg.moe_w8a16_gemm1(to_dev_act(xb, act), W.w13, W.s13, s, b, n, bm, k, a)
    torch.cuda.synchronize()
    sr, br, nr = oracle.align_block(ids_ref, E, bm)
    raw = a.cpu().numpy().view(np.uint8)
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    qh = raw[:cap * I].view(np.int8).reshape(cap, I).astype(np.int64)
    ql = raw[up(cap * I):up(cap * I) + cap * I].view(np.int8).reshape(cap, I).astype(np.int64)
    o = 2 * up(cap * I)
    qs = raw[o:o + cap * (I // 128) * 4].view(np.float32).reshape(cap, I // 128).astype(np.float64)
    xf = oracle.act_bits_to_f64(xb, act)
    checked = 0
    for blk in range(nr // bm):
        W13 = oracle.dequant_int8_rows(W.q13[br[blk]], W.hs13[br[blk]])
        rows = sr[blk * bm:(blk + 1) * bm]
        for r_local in range(16 * ((np.sum(rows < T * k) + 15) // 16)):
            r = blk * bm + r_local
            f = rows[r_local]
            if f >= T * k:
                assert np.all(qh[r] == 0) and np.all(ql[r] == 0) and np.all(qs[r] == 0.0)
                continue
            ref = oracle.moe_expert_intermediate(xf[f // k][None], W13, I)[0]
            gmax = np.abs(ref).reshape(-1, 128).max(axis=1)
            assert np.allclose(qs[r], gmax / 32639.0, rtol=1e-4, atol=0.0), (blk, r_local)
            sc = np.repeat(qs[r], 128)
            vq = sc * (256.0 * qh[r] + ql[r])
            tol = 0.51 * sc + 2e-5 * np.abs(ref).max() + 1e-4 * np.abs(ref)
            assert np.all(np.abs(vq - ref) <= tol), (blk, r_local, np.abs(vq - ref).max())
            checked += 1
    assert checked == T * k


@pytest.mark.parametrize("act,bm", [("bf16", 16), ("fp16", 32), ("fp16", 16), ("bf16", 64), ("bf16", 48)])
def test_gemm1_intermediate(act, bm):
    E, k, H, I, T = 8, 2, 384, 640, 29
    log(f"[gemm1] act={act} bm={bm} E={E} H={H} I={I} T={T}")
    W = small_w8(E, H, I, seed=3)
    assert W.mismatch == 0
    xb = synthetic.random_activations(T, H, act, seed=4)
    logits = synthetic.random_logits(T, E, seed=5)
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    cap = pkg.moe_align_capacity(T, k, E, bm)
    s = torch.empty(cap, dtype=torch.int32, device=DEV)
    b = torch.empty(cap // bm, dtype=torch.int32, device=DEV)
    n = torch.empty(1, dtype=torch.int32, device=DEV)
    pkg.moe_align_block(ti, E, bm, s, b, n)
    nbytes = pkg.moe_w8a16_intermediate_bytes(T, H, I, E, k, bm)
    a = torch.full(((nbytes + 1) // 2,), 0x7FC0, dtype=torch.int16, device=DEV)   # bf16 NaN fill
    x = to_dev_act(xb, act)
    pkg.moe_w8a16_gemm1(x, W.w13, W.s13, s, b, n, bm, k, a)
    pkg.moe_w8a16_requant(a, T, I, E, k, s, n, bm)
    torch.cuda.synchronize()
    sr, br, nr = oracle.align_block(ids_ref, E, bm)
    raw = a.cpu().numpy().view(np.uint8)
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    xf = oracle.act_bits_to_f64(xb, act)
    if bm in (16, 32):
        # GEMM1 writes the 16-bit fixed-point form itself, groups of 64 columns, at offset 0
        qh = raw[:cap * I].view(np.int8).reshape(cap, I).astype(np.int64)
        ql = raw[up(cap * I):up(cap * I) + cap * I].view(np.int8).reshape(cap, I).astype(np.int64)
        o = 2 * up(cap * I)
        qs = raw[o:o + cap * (I // 64) * 4].view(np.float32).reshape(cap, I // 64).astype(np.float64)
        assert qh.min() >= -127 and qh.max() <= 127
        checked = 0
        for blk in range(nr // bm):
            W13 = oracle.dequant_int8_rows(W.q13[br[blk]], W.hs13[br[blk]])
            rows = sr[blk * bm:(blk + 1) * bm]
            for r_local in range(16 * ((np.sum(rows < T * k) + 15) // 16)):
                r = blk * bm + r_local
                f = rows[r_local]
                if f >= T * k:
                    assert np.all(qh[r] == 0) and np.all(ql[r] == 0) and np.all(qs[r] == 0.0)
                    continue
                ref = oracle.moe_expert_intermediate(xf[f // k][None], W13, I)[0]
                gmax = np.abs(ref).reshape(-1, 64).max(axis=1)
                assert np.allclose(qs[r], gmax / 32639.0, rtol=1e-4, atol=0.0), (blk, r_local)
                sc = np.repeat(qs[r], 64)
                vq = sc * (256.0 * qh[r] + ql[r])
                tol = 0.51 * sc + 2e-5 * np.abs(ref).max() + 1e-4 * np.abs(ref)
                assert np.all(np.abs(vq - ref) <= tol), (blk, r_local, np.abs(vq - ref).max())
                checked += 1
        assert checked == T * k
        return
    planes = raw[:4 * cap * I].view(np.uint16).reshape(2, cap, I)
    a_g = oracle.bf16_bits_to_f64(planes[0]) + oracle.bf16_bits_to_f64(planes[1])
    if 32 < bm <= 64:
        # the 16-bit fixed-point form after the planes: v ~= s * (256 hi + lo) per (row, 128 columns)
        o = up(4 * cap * I)
        qh = raw[o:o + cap * I].view(np.int8).reshape(cap, I).astype(np.int64)
        o += up(cap * I)
        ql = raw[o:o + cap * I].view(np.int8).reshape(cap, I).astype(np.int64)
        o += up(cap * I)
        qs = raw[o:o + cap * (I // 128) * 4].view(np.float32).reshape(cap, I // 128).astype(np.float64)
        assert qh.min() >= -127 and qh.max() <= 127
        for blk in range(nr // bm):
            rows = sr[blk * bm:(blk + 1) * bm]
            for r_local in range(16 * ((np.sum(rows < T * k) + 15) // 16)):
                r = blk * bm + r_local
                sc = np.repeat(qs[r], 128)
                gmax = np.abs(a_g[r]).reshape(-1, 128).max(axis=1)
                assert np.allclose(qs[r], gmax / 32639.0, rtol=1e-6, atol=0.0), (blk, r_local)
                vq = sc * (256.0 * qh[r] + ql[r])
                assert np.all(np.abs(vq - a_g[r]) <= 0.51 * sc + 1e-30), (blk, r_local)
    for blk in range(nr // bm):
        e = br[blk]
        W13 = oracle.dequant_int8_rows(W.q13[e], W.hs13[e])
        rows = sr[blk * bm:(blk + 1) * bm]
        for r_local, f in enumerate(rows):
            r = blk * bm + r_local
            if f >= T * k:
                if r_local < 16 * ((np.sum(rows < T * k) + 15) // 16):
                    assert np.all(a_g[r] == 0.0)   # padding rows of a computed 16-row group
                continue
            ref = oracle.moe_expert_intermediate(xf[f // k][None], W13, I)[0]
            err = np.abs(a_g[r] - ref)
            assert np.all(err <= 2e-5 * np.abs(ref).max() + 1e-4 * np.abs(ref)), (blk, f, err.max())


@pytest.mark.parametrize("splits", [1, 2, 3])
def test_gemm2_blocks_of_256_splits(splits):
    # the stage calls at 256-row blocks (fixed-point intermediate, integer
    # GEMM2) with K cut into 1, 2 or 3 parts of whole 128-wide groups (I/128 =
    # 3, so two parts are uneven); the combined output against the oracle layer
    E, k, H, I, T, bm = 4, 2, 512, 384, 300, 256
    log(f"[gemm2 256 splits] splits={splits} E={E} H={H} I={I} T={T}")
    W = small_w8(E, H, I, seed=21)
    xb = synthetic.random_activations(T, H, "bf16", seed=22)
    logits = synthetic.random_logits(T, E, seed=23)
    tw, ti, w_ref, ids_ref = route_both(logits, k)
    cap = pkg.moe_align_capacity(T, k, E, bm)
    s = torch.empty(cap, dtype=torch.int32, device=DEV)
    b = torch.empty(cap // bm, dtype=torch.int32, device=DEV)
    n = torch.empty(1, dtype=torch.int32, device=DEV)
    pkg.moe_align_block(ti, E, bm, s, b, n)
    nbytes = pkg.moe_w8a16_intermediate_bytes(T, H, I, E, k, bm)
    a = torch.zeros(((nbytes + 1) // 2,), dtype=torch.int16, device=DEV)
    pkg.moe_w8a16_gemm1(to_dev_act(xb, "bf16"), W.w13, W.s13, s, b, n, bm, k, a)
    y = torch.full((splits, T * k, H), float("nan"), dtype=torch.float32, device=DEV)
    pkg.moe_w8a16_gemm2(a, T, k, W.w2, W.s2, s, b, n, bm, splits, y)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    pkg.moe_combine_topk(y, splits, tw, ti, E, out)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any(), "every part writes every valid row"
    got = out.float().cpu().numpy().astype(np.float64)
    ok, detail = oracle.layer_within_tolerance(got, oracle.moe_forward_w8(
        oracle.bf16_bits_to_f64(xb), W.q13, W.hs13, W.q2, W.hs2, w_ref, ids_ref))
    assert ok, f"splits={splits}: {detail}"


# (T, k, splits, H, act): every register shape of the few-token combine
# (k <= 2 with 1, 2, 3-4 and 5-16 parts; k <= 8 with 1, 2, 3-4 parts), k = 1,
# the slots-over-waves kernel for more partials (k = 3 with 5 parts, k = 6 with
# 8 as fine-grained decode at one token, k = 16 with 16 at its limits, 96
# groups per token so that a workgroup straddles two tokens), and the general
# kernel (k = 17; 17 parts; more than 256 workgroups with one part and with 12)
@pytest.mark.parametrize("T,k,splits,H,act", [
    (1, 2, 1, 4096, "bf16"), (3, 2, 2, 4096, "bf16"), (1, 2, 3, 4096, "fp16"), (1, 2, 16, 4096, "bf16"),
    (5, 2, 9, 512, "bf16"), (1, 1, 16, 512, "fp16"), (2, 6, 1, 2048, "bf16"), (4, 8, 2, 2048, "fp16"),
    (3, 6, 4, 2048, "bf16"), (2, 3, 5, 512, "bf16"), (1, 6, 8, 2048, "bf16"), (1, 16, 16, 1024, "fp16"),
    (3, 12, 9, 384, "bf16"), (2, 17, 2, 512, "bf16"), (2, 4, 17, 256, "fp16"), (40, 2, 12, 4096, "bf16"),
    (300, 2, 1, 4096, "bf16"), (70, 2, 12, 4096, "fp16")])
def test_combine_topk(T, k, splits, H, act):
    log(f"[combine] T={T} k={k} splits={splits} H={H} act={act}")
    E = 8
    rng = np.random.default_rng(T * 1000 + k * 100 + splits)
    y = rng.standard_normal((splits, T * k, H)).astype(np.float32)
    w = rng.uniform(0.0, 1.0, (T, k)).astype(np.float32)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    ids[0, k - 1] = -1                     # a dropped assignment
    if T > 1:
        ids[1, 0] = E                      # an id past the experts
    out = torch.empty(T, H, dtype=torch.bfloat16 if act == "bf16" else torch.float16, device=DEV)
    pkg.moe_combine_topk(torch.from_numpy(y).to(DEV), splits, torch.from_numpy(w).to(DEV),
                         torch.from_numpy(ids).to(DEV), E, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.combine_topk(y, w, ids, E)
    # fp32 sums of splits parts and k weighted slots (relative error of each
    # step 2^-24, bounded by the sum of magnitudes), then one rounding to the
    # output type (half an ulp: 2^-8 relative for bf16, 2^-11 for fp16)
    valid = ((ids >= 0) & (ids < E)).astype(np.float64)
    mag = np.einsum("tj,tjh->th", np.abs(w) * valid, np.abs(y).sum(axis=0).reshape(T, k, H))
    u_out = 2.0 ** -8 if act == "bf16" else 2.0 ** -11
    tol = u_out * np.abs(ref) + (splits + k + 1) * 2.0 ** -23 * mag + 2.0 ** -24
    err = np.abs(got - ref)
    assert np.all(err <= tol), (float(err.max()), float((err - tol).max()))
