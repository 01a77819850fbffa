"""The seeded input recipe: bf16 rounding agrees with torch's round-to-nearest-even,
draw order and shapes are stable."""
import numpy as np
import pytest

from gla_inputs import CONFIGS, generate, round_to_bf16_bits, bf16_bits_to_f64, logsigmoid


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 0.0])])
    x32 = x.astype(np.float32)
    mine = round_to_bf16_bits(x32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(bf16_bits_to_f64(mine), torch.from_numpy(x32).to(torch.bfloat16).double().numpy())


def test_logsigmoid():
    x = np.array([-800.0, -3.0, 0.0, 2.0, 800.0])
    ref = np.array([-800.0, np.log(1 / (1 + np.exp(3.0))), np.log(0.5), np.log(1 / (1 + np.exp(-2.0))), 0.0])
    assert np.allclose(logsigmoid(x), ref, rtol=1e-14, atol=1e-300)


def test_generate_shapes_and_exactness():
    cfg = CONFIGS["tiny_f32"]
    d = generate(cfg)
    assert d["q"].shape == (1, 1, 256, 64) and d["v"].shape == (1, 1, 256, 64)
    assert np.all(d["log_alpha"] <= 0)
    assert np.array_equal(d["q_store"].astype(np.float64), d["q"])
    c2 = CONFIGS["gla340m_t2k"].replace(T=64)
    d2 = generate(c2)
    assert d2["q_store"].dtype == np.uint16
    assert np.array_equal(bf16_bits_to_f64(d2["k_store"]), d2["k"])
    # seeded: same draws twice
    assert np.array_equal(generate(c2)["v_store"], d2["v_store"])
