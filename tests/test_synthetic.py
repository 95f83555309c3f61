"""The seeded input generator: deterministic, right shapes and distributions."""
import numpy as np

from weight_quantized_mixture_amd import synthetic


def test_deterministic_and_shapes():
    wl = synthetic.WORKLOADS["tiny"]
    a = synthetic.activations(wl, 16, 0)
    b = synthetic.activations(wl, 16, 0)
    assert a.dtype == np.uint16 and a.shape == (16, 256)
    np.testing.assert_array_equal(a, b)
    w = synthetic.expert_master(wl, "w13", 3)
    assert w.shape == (1024, 256) and w.dtype == np.float32
    np.testing.assert_array_equal(w, synthetic.expert_master(wl, "w13", 3))
    assert not np.array_equal(w, synthetic.expert_master(wl, "w13", 4))
    assert abs(float(w.std()) - 0.02) < 1e-3
    assert synthetic.expert_master(wl, "w2", 0).shape == (256, 512)


def test_bf16_rounding_half_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e38], np.float32)
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125 -> even (1.0); 1 + 3*2^-8 -> 1.015625
    bits = synthetic.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(back[:4], np.array([1.0, 1.0, 1.015625, -2.5], np.float32))


def test_bias_shapes_loads():
    fg = synthetic.WORKLOADS["fine_grained"]
    l = synthetic.router_logits(fg, 512)
    assert l.shape == (512, 64)
    top = np.argmax(l, axis=1)
    assert (top == 0).mean() > 0.5          # Zipf bias: expert 0 dominates
    pf = synthetic.WORKLOADS["mixtral_prefill"]
    assert synthetic.expert_bias(pf).std() > 0.1
