"""The seeded input generators (CPU only)."""
import numpy as np
import torch

from selective_state_space_65_amd import inputs


def test_same_seed_same_bytes():
    a = inputs.make_scan_inputs(2, 20, 4, 33, io="bf16", seed=5, h0=True)
    b = inputs.make_scan_inputs(2, 20, 4, 33, io="bf16", seed=5, h0=True)
    for k in ("u", "delta", "A", "B", "C", "D", "z", "delta_bias", "h0"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    c = inputs.make_scan_inputs(2, 20, 4, 33, io="bf16", seed=6, h0=True)
    assert not np.array_equal(a.u, c.u)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, 3.3895314e38], np.float32)]).astype(np.float32)
    ours = inputs.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(inputs.round_bf16(np.array([np.nan], np.float32))[0])


def test_distributions():
    x = inputs.scan_config(0)
    b, d, n, l = x.shape
    assert (b, d, n, l) == (1, 16, 4, 64)
    assert np.array_equal(x.A, np.tile(-(np.arange(4) + 1.0), (16, 1)).astype(np.float32))
    dt = np.log1p(np.exp(x.delta_bias.astype(np.float64)))
    assert dt.min() >= 1e-3 * 0.999 and dt.max() <= 0.1 * 1.001
    assert np.all(x.D == 1.0) and x.z is not None and x.softplus
    big = inputs.make_scan_inputs(1, 64, 16, 4096, seed=1)
    assert abs(big.u.std() - 1.0) < 0.01 and abs(big.delta.std() - 0.5) < 0.01


def test_bf16_config_values_are_bf16():
    x = inputs.make_scan_inputs(2, 8, 16, 64, io="bf16", seed=3)
    for k in ("u", "delta", "z", "B", "C"):
        v = getattr(x, k).view(np.uint32)
        assert np.all((v & 0xFFFF) == 0), k


def test_decode_steps_are_seeded():
    dec = inputs.decode_config(batch=4, dim=8, steps=3)
    s0, s0b, s1 = dec.step(0), dec.step(0), dec.step(1)
    assert all(np.array_equal(s0[k], s0b[k]) for k in s0)
    assert not np.array_equal(s0["u"], s1["u"])
    assert abs(float(inputs.decode_config(batch=64, dim=512).state0.std()) - 0.1) < 0.01


def test_sample_channels():
    ch = inputs.sample_channels(4, 100, 10, seed=1)
    assert len(ch) == 10 and ch[0] == (0, 0) and ch[-1] == (3, 99) and len(set(ch)) == 10


def test_test_recipe_varies_A_and_D_per_channel():
    x = inputs.make_scan_inputs(2, 300, 16, 8, seed=9)
    assert np.unique(x.A[:, 0]).size == 300 and np.unique(x.D).size == 300
    # Each A row is a positive multiple of -(n + 1), the multiple in [1/2, 2].
    s = x.A[:, 0] / -1.0
    assert np.allclose(x.A, -(np.arange(16) + 1.0)[None, :] * s[:, None], rtol=1e-6)
    assert s.min() >= 0.5 and s.max() <= 2.0
    # The other tensors are those of the workload recipe with the same seed.
    w = inputs.make_scan_inputs(2, 300, 16, 8, seed=9, channel_params_kind="workload")
    for k in ("u", "delta", "z", "B", "C", "delta_bias"):
        assert np.array_equal(getattr(x, k), getattr(w, k)), k
    assert np.all(w.D == 1.0) and np.unique(w.A[:, 0]).size == 1
    dec = inputs.decode_config(batch=2, dim=50, steps=1, channel_params_kind="varied")
    assert np.unique(dec.D).size == 50 and np.unique(dec.A[:, 3]).size == 50
