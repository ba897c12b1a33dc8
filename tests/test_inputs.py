"""The seeded input generator: determinism, storage format and recipe."""
import numpy as np
import torch

import moe_inputs as mi


def test_bf16_storage_matches_torch_cast():
    a = (np.random.default_rng(0).standard_normal(50000) * 7).astype(np.float32)
    bits = mi.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    np.testing.assert_array_equal(mi.bf16_bits_to_f32(bits),
                                  torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_per_expert():
    cfg = mi.small_config(d_model=64, d_ff=128, n_experts=5, dtype="bf16")
    a = mi.make_layer(cfg, workers=1)
    b = mi.make_layer(cfg, workers=4)
    for name in ("w_router", "w_gate", "w_up", "w_down"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    g3, u3, d3 = mi.make_expert(cfg, 3)
    np.testing.assert_array_equal(a.w_gate[3], g3)
    np.testing.assert_array_equal(a.w_down[3], d3)


def test_decode_x_is_prefill_prefix():
    pre, dec = mi.CONFIGS["dsv3_prefill"], mi.CONFIGS["dsv3_decode"]
    small_pre = mi.with_(pre, n_tokens=130, d_model=64)
    small_dec = mi.with_(dec, d_model=64)
    np.testing.assert_array_equal(mi.make_x(small_pre)[:64], mi.make_x(small_dec))


def test_recipe_statistics():
    cfg = mi.small_config(d_model=256, d_ff=512, n_experts=4, n_tokens=256, dtype="f32")
    lay, x = mi.make_layer(cfg), mi.make_x(cfg)
    assert abs(x.std() - 1.0) < 0.01
    assert abs(lay.w_router.std() * 16 - 1.0) < 0.05          # std = d^-1/2
    assert abs(lay.w_down.std() * np.sqrt(512) - 1.0) < 0.01  # std = d_ff^-1/2


def test_biases():
    sw = mi.with_(mi.CONFIGS["switch_cap"], d_model=64)
    lb, sb = mi.make_biases(sw)
    assert sb is None and lb.dtype == np.float32
    np.testing.assert_allclose(np.sort(lb)[::-1], 1.5 * np.log(1.0 / np.arange(1, 129)), rtol=1e-6)
    assert sw.capacity == 160
    _, sb2 = mi.make_biases(mi.CONFIGS["dsv3_prefill"])
    assert sb2.shape == (256,) and np.all(np.abs(sb2) <= 0.1)
