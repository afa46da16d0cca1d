"""GPU parity of ssd_step_multi: K pre-staged decode steps with the state on chip, against the
oracle's token recurrence (the same definition the forward is checked against) and against K
single-step calls."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, make_forward_inputs, make_step_inputs, seed_for
from tests.gpu_util import assert_close_state, assert_close_y, dev, host, rel_l2

pytestmark = pytest.mark.gpu

# (b, K, H, P, N, G, dtype): on-chip shapes over the register-block sizes (P/16 rows x N/16
# columns per thread), ragged step blocks (K not a multiple of 16), and shapes that run one step
# kernel per token (N = 32: fewer than four columns per thread; 128 x 256: over 64 per thread)
CASES = [
    (3, 37, 4, 64, 128, 2, "bf16"),
    (2, 16, 3, 64, 128, 1, "f32"),
    (1, 5, 2, 16, 64, 1, "bf16"),
    (2, 33, 2, 32, 256, 2, "bf16"),
    (1, 20, 2, 128, 64, 1, "f32"),
    (1, 19, 3, 256, 64, 3, "bf16"),
    (1, 12, 2, 48, 64, 1, "bf16"),
    (1, 3, 1, 16, 1024, 1, "f32"),
    (2, 7, 2, 48, 32, 1, "bf16"),
    (1, 9, 2, 128, 256, 1, "f32"),
    (4, 1, 2, 64, 64, 1, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "b{}_K{}_H{}_P{}_N{}_G{}_{}".format(*c))
def test_step_multi_matches_oracle(gpu_ssd, case):
    b, K, H, P, N, G, dtype = case
    fi = make_forward_inputs(b, K, H, P, N, G, dtype, 130, h0_std=0.3)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    S = dev(fi.h0)
    y = gpu_ssd.step_multi(S, dev(fi.x, dtype), dev(fi.dt, dtype), dev(fi.A), dev(fi.B, dtype), dev(fi.C, dtype),
                           dev(fi.D))
    torch.cuda.synchronize()
    assert_close_y(host(y), ref["y"], dtype)
    assert_close_state(host(S), ref["final"])


@pytest.mark.parametrize("mode", ["long_memory", "extreme", "per_head_bias", "zero"])
def test_step_multi_dt_modes(gpu_ssd, mode):
    """Tiny steps (long memory), huge steps (decay underflow within a block of steps), spread steps and
    zero steps, against the oracle."""
    b, K, H, P, N, G = 2, 40, 4, 64, 128, 1
    a_mode = "minus_one" if mode == "long_memory" else "config"
    fi = make_forward_inputs(b, K, H, P, N, G, "f32", 133, dt_mode=mode, a_mode=a_mode, h0_std=0.5)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    S = dev(fi.h0)
    y = gpu_ssd.step_multi(S, dev(fi.x), dev(fi.dt), dev(fi.A), dev(fi.B), dev(fi.C), dev(fi.D))
    torch.cuda.synchronize()
    assert_close_y(host(y), ref["y"], "f32")
    assert_close_state(host(S), ref["final"])


def test_step_multi_equals_single_steps(gpu_ssd):
    """One K-step call and K ssd_step calls on the slices [:, k] give the same state and outputs."""
    b, K, H, P, N, G = 2, 24, 4, 64, 128, 1
    fi = make_forward_inputs(b, K, H, P, N, G, "f32", 131, h0_std=0.5)
    S1, S2 = dev(fi.h0), dev(fi.h0)
    x, dt, B, C = dev(fi.x), dev(fi.dt), dev(fi.B), dev(fi.C)
    A, D = dev(fi.A), dev(fi.D)
    ym = gpu_ssd.step_multi(S1, x, dt, A, B, C, D)
    ys = torch.stack([gpu_ssd.step(S2, x[:, k].contiguous(), dt[:, k].contiguous(), A, B[:, k].contiguous(),
                                   C[:, k].contiguous(), D) for k in range(K)], dim=1)
    torch.cuda.synchronize()
    # the state update is the same elementwise recurrence; y differs only in summation order
    assert rel_l2(host(S1), host(S2)) < 1e-6
    assert rel_l2(host(ym), host(ys)) < 1e-5


def test_step_multi_zero_steps_and_no_d(gpu_ssd):
    fi = make_forward_inputs(2, 12, 2, 64, 64, 1, "bf16", 132, h0_std=0.3, with_D=False)
    S = dev(fi.h0)
    S0 = S.clone()
    x = dev(fi.x, "bf16")
    y0 = gpu_ssd.step_multi(S, x[:, :0].contiguous(), dev(fi.dt, "bf16")[:, :0].contiguous(), dev(fi.A),
                            dev(fi.B, "bf16")[:, :0].contiguous(), dev(fi.C, "bf16")[:, :0].contiguous(), None)
    torch.cuda.synchronize()
    assert y0.shape[1] == 0 and torch.equal(S, S0)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, None, fi.h0)
    y = gpu_ssd.step_multi(S, x, dev(fi.dt, "bf16"), dev(fi.A), dev(fi.B, "bf16"), dev(fi.C, "bf16"), None)
    torch.cuda.synchronize()
    assert_close_y(host(y), ref["y"], "bf16")
    assert_close_state(host(S), ref["final"])


def test_cfg4_multi_step_decode(gpu_ssd):
    """The 2.7B decode shape (b=64, H=80, P=64, N=128), 64 steps in one call, against the oracle's
    step-by-step recurrence (y of every step and the final state)."""
    cfg = CONFIGS["cfg4"]
    si = make_step_inputs(cfg["batch"], cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"],
                          steps=cfg["steps"], dtype=cfg["dtype"], seed=seed_for("cfg4"))
    S = dev(si.state0)
    x = torch.stack([dev(si.x[k], "bf16") for k in range(64)], dim=1).contiguous()
    dt = torch.stack([dev(si.dt[k], "bf16") for k in range(64)], dim=1).contiguous()
    B = torch.stack([dev(si.B[k], "bf16") for k in range(64)], dim=1).contiguous()
    C = torch.stack([dev(si.C[k], "bf16") for k in range(64)], dim=1).contiguous()
    y = gpu_ssd.step_multi(S, x, dt, dev(si.A), B, C, dev(si.D))
    torch.cuda.synchronize()
    ref_state = np.array(si.state0, dtype=np.float64)
    ys = []
    for k in range(64):
        ys.append(oracle.step(ref_state, si.x[k], si.dt[k], si.A, si.B[k], si.C[k], si.D))
    assert_close_y(host(y), np.stack(ys, axis=1), "bf16")
    assert_close_state(host(S), ref_state)


def test_step_chain_in_a_graph(gpu_ssd):
    """ssd_step launches captured in one graph replay to the eager result, replay after replay."""
    b, K, H, P, N, G = 4, 8, 6, 64, 128, 1
    fi = make_forward_inputs(b, K, H, P, N, G, "bf16", 133, h0_std=0.3)
    S0 = dev(fi.h0)
    xs = [dev(fi.x[:, k], "bf16") for k in range(K)]
    dts = [dev(fi.dt[:, k], "bf16") for k in range(K)]
    Bs = [dev(fi.B[:, k], "bf16") for k in range(K)]
    Cs = [dev(fi.C[:, k], "bf16") for k in range(K)]
    A, D = dev(fi.A), dev(fi.D)
    S = S0.clone()
    ye = torch.stack([gpu_ssd.step(S, xs[k], dts[k], A, Bs[k], Cs[k], D) for k in range(K)], dim=1)
    S_eager = S.clone()
    Sg = S0.clone()
    yg = [torch.empty_like(xs[0]) for _ in range(K)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(K):
            gpu_ssd.step(Sg, xs[k], dts[k], A, Bs[k], Cs[k], D, y=yg[k])
    for rep in range(3):
        Sg.copy_(S0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(Sg, S_eager), f"replay {rep}: state"
        assert torch.equal(torch.stack(yg, dim=1), ye), f"replay {rep}: y"
        _ = (S_eager * 2).sum().item()  # eager work between replays
