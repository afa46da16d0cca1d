"""GPU parity of the dt front-end (*_ex calls): per-head bias, softplus, clamp and the
zero-order-hold input step, against the oracle's front-end followed by its recurrence."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_05_amd as ssd_mod
import oracle
from synth import make_forward_inputs, round_to
from tests.gpu_util import assert_close_state, assert_close_y, dev, host, rel_l2

pytestmark = pytest.mark.gpu

MODES = {
    "softplus_bias": dict(softplus=True, zoh=False, clamp=None),
    "softplus_bias_clamp": dict(softplus=True, zoh=False, clamp=(2e-3, 0.05)),
    "zoh": dict(softplus=False, zoh=True, clamp=None),
    "all": dict(softplus=True, zoh=True, clamp=(1e-3, 0.08)),
}


def _raw_dt(fi, mode, dtype, seed):
    """A raw step for the front-end: pre-softplus values around softplus^-1(0.01) when softplus is on,
    else the workload's positive dt; rounded to the device dtype, as the device sees it."""
    rng = np.random.default_rng(seed)
    H = fi.dt.shape[-1]
    bias = rng.normal(0.0, 0.5, H)
    if MODES[mode]["softplus"]:
        raw = rng.normal(-4.6, 1.0, fi.dt.shape)
    else:
        raw = fi.dt * 5.0  # larger steps make the ZOH factor differ visibly from dt
        bias = None
    raw = round_to(raw, dtype)
    bias = None if bias is None else round_to(bias, "f32")
    return raw, bias


def _frontend(mode, bias):
    m = MODES[mode]
    return ssd_mod.Frontend(dt_bias=None if bias is None else dev(bias), softplus=m["softplus"], zoh=m["zoh"],
                            clamp=m["clamp"])


def _oracle_steps(raw, A, bias, mode):
    m = MODES[mode]
    return oracle.dt_frontend(raw, A, bias, softplus=m["softplus"], zoh=m["zoh"], clamp=m["clamp"])


# (b, L, H, P, N, G, dtype, chunk): the fast forward (bf16, P 64, N 128) and the generic one (fp32)
SHAPES = [(2, 700, 4, 64, 128, 2, "bf16", 0), (1, 300, 3, 32, 64, 1, "f32", 64)]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}_L{}_H{}_P{}_N{}_G{}_{}_Q{}".format(*s))
def test_forward_frontend(gpu_ssd, shape, mode):
    b, L, H, P, N, G, dtype, chunk = shape
    fi = make_forward_inputs(b, L, H, P, N, G, dtype, 150, h0_std=0.3)
    raw, bias = _raw_dt(fi, mode, dtype, 151)
    dec, inp = _oracle_steps(raw, fi.A, bias, mode)
    ref = oracle.forward(fi.x, dec, fi.A, fi.B, fi.C, fi.D, fi.h0, dt_in=inp)
    y, fin = gpu_ssd.forward(dev(fi.x, dtype), dev(raw, dtype), dev(fi.A), dev(fi.B, dtype), dev(fi.C, dtype),
                             dev(fi.D), dev(fi.h0), chunk=chunk, frontend=_frontend(mode, bias))
    torch.cuda.synchronize()
    assert_close_y(host(y), ref["y"], dtype)
    assert_close_state(host(fin), ref["final"])
    if mode == "zoh":  # the ZOH factor visibly changes the result against the plain step
        plain = oracle.forward(fi.x, dec, fi.A, fi.B, fi.C, fi.D, fi.h0)
        assert rel_l2(plain["final"], ref["final"]) > 1e-2


def test_forward_frontend_long(gpu_ssd):
    """Above 2^20 token-heads the fast forward keeps its decay pass (the front-end applied there) instead of
    forming the decays in the chunk kernels: every front-end option at once, against the oracle on every head."""
    b, L, H, P, N, G, dtype, chunk = 1, 8256, 128, 64, 64, 2, "bf16", 0  # 1,056,768 token-heads
    mode = "all"
    fi = make_forward_inputs(b, L, H, P, N, G, dtype, 155, h0_std=0.3)
    raw, bias = _raw_dt(fi, mode, dtype, 156)
    dec, inp = _oracle_steps(raw, fi.A, bias, mode)
    ref = oracle.forward(fi.x, dec, fi.A, fi.B, fi.C, fi.D, fi.h0, dt_in=inp)
    y, fin = gpu_ssd.forward(dev(fi.x, dtype), dev(raw, dtype), dev(fi.A), dev(fi.B, dtype), dev(fi.C, dtype),
                             dev(fi.D), dev(fi.h0), chunk=chunk, frontend=_frontend(mode, bias))
    torch.cuda.synchronize()
    assert_close_y(host(y), ref["y"], dtype)
    assert_close_state(host(fin), ref["final"])


@pytest.mark.parametrize("mode", list(MODES))
def test_cumsum_frontend(gpu_ssd, mode):
    fi = make_forward_inputs(2, 200, 5, 16, 16, 1, "f32", 152)
    raw, bias = _raw_dt(fi, mode, "f32", 153)
    dec, inp = _oracle_steps(raw, fi.A, bias, mode)
    want_dt, want_cs = oracle.chunk_cumsum(dec, fi.A, 64, dt_in=inp)
    dt_t, cs = gpu_ssd.chunk_cumsum(dev(raw), dev(fi.A), 64, frontend=_frontend(mode, bias))
    torch.cuda.synchronize()
    assert np.max(np.abs(host(dt_t) - want_dt)) <= 1e-5 * np.max(np.abs(want_dt))
    assert np.max(np.abs(host(cs) - want_cs)) <= 1e-4 * max(1.0, np.max(np.abs(want_cs)))


@pytest.mark.parametrize("mode", list(MODES))
def test_step_and_multi_step_frontend(gpu_ssd, mode):
    b, K, H, P, N, G = 3, 20, 4, 64, 128, 1
    fi = make_forward_inputs(b, K, H, P, N, G, "bf16", 154, h0_std=0.3)
    raw, bias = _raw_dt(fi, mode, "bf16", 155)
    dec, inp = _oracle_steps(raw, fi.A, bias, mode)
    ref = oracle.forward(fi.x, dec, fi.A, fi.B, fi.C, fi.D, fi.h0, dt_in=inp)
    fe = _frontend(mode, bias)
    x, rd, B, C = dev(fi.x, "bf16"), dev(raw, "bf16"), dev(fi.B, "bf16"), dev(fi.C, "bf16")
    A, D = dev(fi.A), dev(fi.D)
    S1 = dev(fi.h0)
    ym = gpu_ssd.step_multi(S1, x, rd, A, B, C, D, frontend=fe)
    S2 = dev(fi.h0)
    ys = torch.stack([gpu_ssd.step(S2, x[:, k].contiguous(), rd[:, k].contiguous(), A, B[:, k].contiguous(),
                                   C[:, k].contiguous(), D, frontend=fe) for k in range(K)], dim=1)
    torch.cuda.synchronize()
    for y, S in ((ym, S1), (ys, S2)):
        assert_close_y(host(y), ref["y"], "bf16")
        assert_close_state(host(S), ref["final"])
