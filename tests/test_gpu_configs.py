"""The five benchmark workloads at full size, through ssd_forward / ssd_step, against the oracle.

Every workload is compared over every head and every token: the GPU runs the
whole problem in the launch configuration the benchmark times (chunk = 0, the
library's choice) and the fp64 oracle recomputes all of it.  y is checked by
its global relative L2 error, per (b, t, h) row and per element
(tests/gpu_util.py); the final state element-wise against its RMS.  The largest
point (256K tokens x 32 heads x headdim 64) holds about 4.3 GB per fp64 copy of
x or y on the host, well inside the GPU host's memory, so no head is sampled.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_config_inputs, make_step_inputs, seed_for
from tests.gpu_util import assert_close_state, assert_close_y, dev, host

pytestmark = pytest.mark.gpu


def _forward_parity(gpu_ssd, name, chunk=0):
    fi = make_config_inputs(name)
    print(f"{name}: inputs drawn", flush=True)
    y, fin = gpu_ssd.forward(dev(fi.x, fi.dtype), dev(fi.dt, fi.dtype), dev(fi.A), dev(fi.B, fi.dtype),
                             dev(fi.C, fi.dtype), dev(fi.D), dev(fi.h0), chunk=chunk)
    torch.cuda.synchronize()
    yg, fg = host(y), host(fin)
    del y, fin
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    del fi
    ey = assert_close_y(yg, ref["y"], CONFIGS[name]["dtype"], f"{name} y")
    es = assert_close_state(fg, ref["final"])
    print(f"{name}: rel L2(y) = {ey:.3e}, max|dS|/RMS = {es:.3e}")


def test_cfg0_tiny_fp32(gpu_ssd):
    """Tiny fp32 case at its own chunk size 64 and at the library's choice."""
    _forward_parity(gpu_ssd, "cfg0", chunk=64)
    _forward_parity(gpu_ssd, "cfg0", chunk=0)


def test_cfg1_130m(gpu_ssd):
    _forward_parity(gpu_ssd, "cfg1")


@pytest.mark.parametrize("name", ["cfg2_1k", "cfg2_4k", "cfg2_16k"])
def test_cfg2_27b_full(gpu_ssd, name):
    _forward_parity(gpu_ssd, name)


def test_cfg2_27b_64k_all_heads(gpu_ssd):
    _forward_parity(gpu_ssd, "cfg2_64k")


@pytest.mark.parametrize("name", [n for n in CONFIGS if n.startswith("cfg3_")])
def test_cfg3_long_context_all_heads(gpu_ssd, name):
    _forward_parity(gpu_ssd, name)


def test_cfg4_decode_64_steps(gpu_ssd):
    """64 consecutive ssd_step calls on the 2.7B shape; every step's y and state are checked."""
    cfg = CONFIGS["cfg4"]
    si = make_step_inputs(cfg["batch"], cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"],
                          steps=cfg["steps"], dtype=cfg["dtype"], seed=seed_for("cfg4"))
    S_ref = si.state0.copy()
    S = dev(si.state0)
    A, D = dev(si.A), dev(si.D)
    ys, ys_ref = [], []
    worst_state = 0.0
    for t in range(cfg["steps"]):
        y = gpu_ssd.step(S, dev(si.x[t], "bf16"), dev(si.dt[t], "bf16"), A, dev(si.B[t], "bf16"),
                         dev(si.C[t], "bf16"), D)
        ys_ref.append(oracle.step(S_ref, si.x[t], si.dt[t], si.A, si.B[t], si.C[t], si.D))
        ys.append(host(y))
        torch.cuda.synchronize()
        worst_state = max(worst_state, assert_close_state(host(S), S_ref, f"state after step {t + 1}"))
    ey = assert_close_y(np.stack(ys), np.stack(ys_ref), "bf16", "y over 64 steps")
    print(f"cfg4: rel L2(y, 64 steps) = {ey:.3e}, worst max|dS|/RMS = {worst_state:.3e}")
