"""The seeded input generators: shapes, value ranges, determinism, bf16 rounding."""

import math

import numpy as np
import torch

import synth


def test_bf16_round_is_rne_like_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-8, 8, 50000),
                        # exact ties between two bf16 neighbours
                        (np.arange(1, 2000, dtype=np.float64) * 2.0 ** -7 + 2.0 ** -8)])
    ours = synth.bf16_round(a)
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)


def test_config_distributions():
    fi = synth.make_config_inputs("cfg1")
    b, L, H, P, N, G = fi.dims
    assert (b, L, H, P, N, G) == (4, 2048, 24, 64, 128, 1)
    lo, hi = 1e-3 * (1 - 2.0 ** -8), 0.1 * (1 + 2.0 ** -8)
    assert fi.dt.min() >= lo and fi.dt.max() <= hi
    # log-uniform: the median of log(dt) sits in the middle of the interval
    mid = 0.5 * (math.log(1e-3) + math.log(0.1))
    assert abs(np.median(np.log(fi.dt)) - mid) < 0.05
    assert np.all(fi.A <= -1.0 + 1e-6) and np.all(fi.A >= -16.0 - 1e-5)
    assert abs(fi.x.std() - 1.0) < 0.01
    assert abs(fi.B.std() * math.sqrt(N) - 1.0) < 0.01
    assert fi.h0 is None
    # every value is exactly representable in the storage dtype
    assert np.array_equal(synth.bf16_round(fi.x), fi.x.astype(np.float32))


def test_seeded_and_deterministic():
    a = synth.make_forward_inputs(1, 64, 2, 8, 8, 1, "bf16", 5)
    b = synth.make_forward_inputs(1, 64, 2, 8, 8, 1, "bf16", 5)
    c = synth.make_forward_inputs(1, 64, 2, 8, 8, 1, "bf16", 6)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.dt, b.dt)
    assert not np.array_equal(a.x, c.x)


def test_step_generator():
    si = synth.make_step_inputs(2, 3, 4, 8, 1, steps=5, seed=4)
    assert si.state0.shape == (2, 3, 4, 8)
    assert si.x.shape == (5, 2, 3, 4) and si.dt.shape == (5, 2, 3) and si.B.shape == (5, 2, 1, 8)
    assert abs(si.state0.std() - 0.1) < 0.05


def test_seeds_follow_the_rule():
    assert synth.seed_for("cfg0") == 0 and synth.seed_for("cfg4") == 4
    assert synth.seed_for("cfg3_256k_n512") == 3000 + 10 * 18 + 9


def test_bursts_mode():
    """Runs of very large steps (0.5 to 2) between the workload's log-uniform ones, per sequence."""
    a = synth.make_forward_inputs(2, 3000, 3, 8, 8, 1, "f32", 9, dt_mode="bursts")
    b = synth.make_forward_inputs(2, 3000, 3, 8, 8, 1, "f32", 9, dt_mode="bursts")
    assert np.array_equal(a.dt, b.dt)
    big = a.dt >= 0.5
    assert a.dt.min() >= 1e-3 * (1 - 1e-6) and a.dt.max() <= 2.0
    assert np.all((a.dt[~big] <= 0.1 * (1 + 1e-6)))
    # every (batch row, head) sequence holds bursts, and bursts are runs (not isolated tokens)
    assert big.any(axis=1).all()
    frac = big.mean()
    assert 0.05 < frac < 0.5
    starts = big[:, 1:] & ~big[:, :-1]
    assert big.sum() / max(starts.sum(), 1) >= 15
