"""The seeded input generator: determinism, head-subset consistency, bf16 exactness."""
import numpy as np

from synth import CONFIGS, generate, to_bf16_bits, bf16_bits_to_f32


def test_deterministic_and_head_subset():
    cfg = CONFIGS["small"].with_(grid=(2, 8, 16), heads=4)
    a = generate(cfg, seed=0)
    b = generate(cfg, seed=0)
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["v"], b["v"])
    sub = generate(cfg, seed=0, heads=[2])
    assert np.array_equal(sub["q"][0, 0], a["q"][0, 2])
    assert np.array_equal(sub["k"][0, 0], a["k"][0, 2])
    c = generate(cfg, seed=1)
    assert not np.array_equal(a["q"], c["q"])


def test_bf16_rounding_and_shapes():
    cfg = CONFIGS["small"].with_(grid=(2, 4, 8))
    g = generate(cfg)
    assert g["q"].shape == (1, 12, 64, 64)
    assert np.array_equal(bf16_bits_to_f32(g["bits"]["k"]), g["k"])
    x = np.array([1.0, 1.00390625, 1.005859375, -3.0e-3], np.float32)
    b = to_bf16_bits(x)
    assert b[0] == 0x3F80 and b[1] == 0x3F80   # tie -> even
    assert b[2] == 0x3F81


def test_tiny_is_fp32_and_temperatures():
    g = generate(CONFIGS["tiny"])
    assert g["bits"] is None and g["q"].shape == (1, 2, 256, 64)
    g3 = generate(CONFIGS["wan_like"].with_(grid=(1, 2, 8)), heads=[0])
    assert np.all((g3["temps"] >= 0.5) & (g3["temps"] <= 2.0))


def test_drift_step_is_a_seeded_small_move():
    from synth import CONFIGS, drift_step, generate
    cfg = CONFIGS["small"].with_(heads=2)
    g = generate(cfg)
    a = drift_step(g, cfg, 1, 0.05)
    b = drift_step(g, cfg, 1, 0.05)
    c = drift_step(g, cfg, 2, 0.05)
    for n in ("q", "k", "v"):
        assert np.array_equal(a["bits"][n], b["bits"][n])
        assert not np.array_equal(a["bits"][n], c["bits"][n])
        d = a[n] - g[n]
        assert abs(float(d.std()) - 0.05) < 0.005          # the walk's step size (plus bf16 rounding)
        assert np.array_equal(to_bf16_bits(a[n]), a["bits"][n])
