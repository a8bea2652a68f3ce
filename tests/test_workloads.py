"""Checks of the seeded synthetic-input generator (no attention arithmetic here)."""
import numpy as np
import torch

from workloads import get_config, make_inputs
from workloads.generator import (bf16_bits_from_f32, cube_order, f32_from_bf16_bits, make_head,
                                 smooth_field, widen)


def test_bf16_bits_match_torch_rounding():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-20, 20, 50000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits_from_f32(x), want)
    np.testing.assert_array_equal(f32_from_bf16_bits(want),
                                  torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_smooth_field_is_standardised_and_smooth():
    f = smooth_field(7, 3, 0, 0, (8, 16, 16), 4)
    assert f.shape == (8, 16, 16, 4)
    np.testing.assert_allclose(f.mean(axis=(0, 1, 2)), 0, atol=1e-5)
    np.testing.assert_allclose(f.std(axis=(0, 1, 2), dtype=np.float64), 1, atol=1e-5)
    # neighbouring cells along x are strongly correlated (blur sigma = 2 cells)
    c = np.corrcoef(f[:, :, :-1, 0].ravel(), f[:, :, 1:, 0].ravel())[0, 1]
    assert c > 0.8


def test_heads_regenerate_identically_and_differ_between_heads():
    cfg = get_config("C2").with_(latent=(4, 8, 8), heads=3)
    full = make_inputs(cfg)
    sub = make_inputs(cfg, heads=[2])
    for key in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(full[key][:, 2:3], sub[key])
    np.testing.assert_array_equal(full["wq"][2:3], sub["wq"])
    assert not np.array_equal(full["q"][0, 0], full["q"][0, 1])
    assert full["q"].dtype == np.uint16 and widen(full["q"]).dtype == np.float64


def test_bias_makes_keys_heavier_and_cube_order_is_a_permutation():
    cfg = get_config("C2").with_(latent=(4, 8, 8), heads=1)
    h = make_head(cfg, 0, 0)
    assert 2.0 < h["k"].std() < 3.2 and 0.9 < h["q"].std() < 1.1
    p = cube_order((4, 8, 8))
    assert sorted(p.tolist()) == list(range(256))
    # the first 64 tokens form the 4x4x4 cube at the origin
    t, rem = np.divmod(p[:64], 64)
    y, x = np.divmod(rem, 8)
    assert t.max() < 4 and y.max() < 4 and x.max() < 4


def test_threaded_generation_gives_the_same_values():
    cfg = get_config("C2").with_(heads=3, latent=(1, 32, 32))
    a = make_inputs(cfg, workers=1)
    b = make_inputs(cfg, workers=3)
    for nm in a:
        assert np.array_equal(a[nm], b[nm]), nm
