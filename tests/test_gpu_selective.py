"""GPU parity of the Mamba-1 selective scan (ssd_selective_scan) against the fp64 oracle.

Inputs come from the seeded generators; sizes span several 64-token tiles, ragged
tails, several sequence segments (the first pass, the carry and the output pass),
groups, every supported state size and both input forms (zero-order hold and
delta * B).  The workload at full size is checked on sampled channels, which the
oracle computes over the whole sequence.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_05_amd as ssd_mod
import oracle
from synth import SELECTIVE_CONFIGS, make_selective_config_inputs, make_selective_inputs, round_to
from tests.gpu_util import assert_close_state, assert_close_y, dev, host

pytestmark = pytest.mark.gpu

# (b, L, Dc, N, G, dtype, segment length, zoh)
CASES = [
    (1, 300, 32, 16, 1, "f32", 0, True),
    (2, 1000, 48, 16, 3, "bf16", 256, True),
    (1, 777, 16, 32, 1, "bf16", 128, False),
    (1, 500, 32, 48, 2, "f32", 64, True),
    (2, 2048, 64, 64, 1, "bf16", 0, True),
    (1, 64, 16, 16, 1, "f32", 0, False),
    (1, 1, 16, 16, 1, "f32", 0, True),
    (3, 4100, 32, 16, 1, "bf16", 0, True),
    (1, 1500, 16, 64, 1, "f32", 192, False),
]


def _ids(c):
    return "b{}_L{}_Dc{}_N{}_G{}_{}_seg{}_{}".format(*c[:7], "zoh" if c[7] else "euler")


def _run(si, zoh, chunk, frontend=None, delta=None):
    fe = frontend if frontend is not None else (ssd_mod.Frontend(zoh=True) if zoh else None)
    y, fin = ssd_mod.selective_scan(dev(si.x, si.dtype), dev(si.delta if delta is None else delta, si.dtype),
                                    dev(si.A), dev(si.B, si.dtype), dev(si.C, si.dtype), dev(si.D), dev(si.h0),
                                    chunk=chunk, frontend=fe)
    torch.cuda.synchronize()
    return host(y), host(fin)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_selective_scan(gpu_ssd, case):
    b, L, Dc, N, G, dtype, chunk, zoh = case
    si = make_selective_inputs(b, L, Dc, N, G, dtype, 200, h0_std=0.3)
    ref = oracle.selective_scan(si.x, si.delta, si.A, si.B, si.C, si.D, si.h0, zoh=zoh)
    y, fin = _run(si, zoh, chunk)
    assert_close_y(y, ref["y"], dtype)
    assert_close_state(fin, ref["final"])


@pytest.mark.parametrize("mode", ["long_memory", "extreme", "zero"])
def test_selective_stress(gpu_ssd, mode):
    """Tiny steps over many segments (the carry matters), huge steps (decay underflow), zero steps."""
    si = make_selective_inputs(1, 3000, 32, 16, 1, "f32", 201, dt_mode=mode, h0_std=0.5)
    ref = oracle.selective_scan(si.x, si.delta, si.A, si.B, si.C, si.D, si.h0, zoh=True)
    y, fin = _run(si, True, 256)
    assert_close_y(y, ref["y"], "f32")
    assert_close_state(fin, ref["final"])


def test_selective_zero_A_and_no_D(gpu_ssd):
    """A[d, n] = 0 takes the zero-order-hold limit (delta); D and h0 may be absent."""
    si = make_selective_inputs(1, 400, 16, 16, 1, "f32", 202, with_D=False)
    si.A[3, 5] = 0.0
    si.A[10, :] = 0.0
    ref = oracle.selective_scan(si.x, si.delta, si.A, si.B, si.C, None, None, zoh=True)
    y, fin = _run(si, True, 128)
    assert_close_y(y, ref["y"], "f32")
    assert_close_state(fin, ref["final"])


@pytest.mark.parametrize("clamp", [None, (2e-3, 0.05)])
def test_selective_frontend(gpu_ssd, clamp):
    """Per-channel bias + softplus (+ clamp) applied to a raw step inside the kernel."""
    si = make_selective_inputs(2, 900, 32, 16, 2, "bf16", 203, h0_std=0.2)
    rng = np.random.default_rng(204)
    raw = round_to(rng.normal(-4.6, 1.0, si.delta.shape), "bf16")
    bias = round_to(rng.normal(0.0, 0.5, 32), "f32")
    delta, _ = oracle.dt_frontend(raw, np.zeros(32), bias, softplus=True, clamp=clamp)
    ref = oracle.selective_scan(si.x, delta, si.A, si.B, si.C, si.D, si.h0, zoh=True)
    fe = ssd_mod.Frontend(dt_bias=dev(bias), softplus=True, zoh=True, clamp=clamp)
    y, fin = _run(si, True, 256, frontend=fe, delta=raw)
    assert_close_y(y, ref["y"], "bf16")
    assert_close_state(fin, ref["final"])


def test_selective_segments_agree(gpu_ssd):
    """The segment length changes nothing beyond rounding (associativity of the recurrence)."""
    si = make_selective_inputs(1, 2500, 32, 32, 1, "f32", 205, dt_mode="long_memory", h0_std=0.4)
    outs = [_run(si, True, c) for c in (0, 64, 640, 2560)]
    for y, fin in outs[1:]:
        assert_close_y(y, outs[0][0], "f32")
        assert_close_state(fin, outs[0][1])


def test_selective_empty(gpu_ssd):
    """L = 0 returns h0 (or zero) as the final state; batch 0 is a no-op."""
    si = make_selective_inputs(2, 1, 16, 16, 1, "f32", 206, h0_std=1.0)
    x = dev(si.x[:, :0])
    y, fin = ssd_mod.selective_scan(x, dev(si.delta[:, :0]), dev(si.A), dev(si.B[:, :0]), dev(si.C[:, :0]),
                                    dev(si.D), dev(si.h0))
    torch.cuda.synchronize()
    assert y.shape[1] == 0 and np.array_equal(host(fin), si.h0)
    y, fin = ssd_mod.selective_scan(x, dev(si.delta[:, :0]), dev(si.A), dev(si.B[:, :0]), dev(si.C[:, :0]))
    torch.cuda.synchronize()
    assert np.all(host(fin) == 0.0)


def test_selective_workload_sampled(gpu_ssd):
    """The benchmark workload at full size, in the launch configuration the benchmark times: every
    channel runs on the GPU, and sampled channels are recomputed by the oracle over the whole
    sequence."""
    name = "mamba1_5120ch_64k"
    cfg = SELECTIVE_CONFIGS[name]
    si = make_selective_config_inputs(name)
    y, fin = _run(si, True, 0)
    chans = np.array([0, 1, 17, 1023, 2500, 4095, 5119])
    ref = oracle.selective_scan(si.x[:, :, chans], si.delta[:, :, chans], si.A[chans], si.B, si.C, si.D[chans],
                                None, zoh=True)
    assert_close_y(y[:, :, chans], ref["y"], cfg["dtype"])
    assert_close_state(fin[:, chans], ref["final"])
