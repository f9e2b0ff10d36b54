"""The seeded generator: determinism, per-head independence, rounding."""
import numpy as np
import torch

from svsa_synth import make_inputs, f32_to_bf16_bits, bf16_bits_to_f32, get_config


def test_deterministic_and_head_subset_consistent():
    a = make_inputs("small", seed=3)
    b = make_inputs("small", seed=3, heads=[5, 1])
    assert np.array_equal(a.q[:, [5, 1]], b.q) and np.array_equal(a.v[:, [5, 1]], b.v)
    assert np.array_equal(a.scales[[5, 1]], b.scales)
    c = make_inputs("small", seed=4)
    assert not np.array_equal(a.q, c.q)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)
    assert np.array_equal(bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).float().numpy())


def test_shapes_and_params():
    t = make_inputs("tiny")
    assert t.q.shape == (1, 1, 256, 64) and t.q32.shape == (1, 1, 256, 64)
    assert np.array_equal(f32_to_bf16_bits(t.q32), t.q)
    cfg = get_config("hv720")
    assert (cfg.N, cfg.nb, cfg.N_pad) == (118800, 1857, 118848)
    assert get_config("wan720").nb == 1182 and get_config("wan480").nb == 512
    w = make_inputs("wan480", heads=[0])
    assert 0.5 <= w.scales[0] <= 3.0 and 0.1 <= w.keep_frac[0] <= 0.5
