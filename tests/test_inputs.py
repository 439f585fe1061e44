"""Checks of the seeded input generator (no GPU)."""
import numpy as np
import torch

from linear_attention_recurrence_03_amd import inputs


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0e-38, 1.00390625, 1.01171875], np.float32)])
    ours = inputs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours, ref)


def test_workload_recipes():
    x = inputs.make(inputs.WORKLOADS[1])
    assert x["q"].shape == (1, 64, 2, 32) and x["state"].shape == (1, 2, 32, 32)
    assert np.all(x["state"] == 0)
    np.testing.assert_allclose(np.linalg.norm(x["k"], axis=-1), 1.0, rtol=1e-5)
    assert np.all(x["g"] <= 0) and np.all((x["beta"] > 0) & (x["beta"] < 1))
    y = inputs.make(inputs.WORKLOADS[1])
    assert all(np.array_equal(x[n], y[n]) for n in x)
    z = inputs.custom(2, 70, 3, 64, dtype="bf16", gate="mixed", beta_std=2.0, seed=1)
    assert np.array_equal(inputs.bf16_round(z["v"]), z["v"])
    frac_strong = np.mean(z["g"] < -2.5)
    assert 0.02 < frac_strong < 0.3


def test_per_sequence_seeds_are_independent_of_slicing():
    wl = inputs.Workload("t", 3, 10, 2, 32, "bf16", "normal", "mixed", 2.0, seed=5,
                         per_seq_seeds=True)
    full = inputs.make(wl)
    one = inputs.make(wl, seq=1)
    for n in full:
        assert np.array_equal(full[n][1:2], one[n])
