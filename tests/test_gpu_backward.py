"""GPU parity of the backward pass (ssd_backward) against the fp64 backward oracle.

Every gradient (dx, ddt, dA, dB, dC, dD, dh0) is compared with the oracle on the same
seeded inputs, at sizes that span several chunks with ragged tails, groups, both io
dtypes, with and without h0, D and a final-state gradient.  The 2.7B-shaped workload
is checked at full size over every head, every gradient.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import mamba_ssd_chunked_05_amd as ssd_mod
import oracle
from synth import make_config_inputs, make_forward_inputs
from tests.gpu_util import Y_TOL, assert_close_state, dev, host, rel_l2

pytestmark = pytest.mark.gpu

# (b, L, H, P, N, G, dtype, chunk, with_h0_and_dfinal)
CASES = [
    (1, 100, 2, 16, 16, 1, "f32", 0, True),
    (2, 300, 4, 32, 64, 2, "f32", 64, True),
    (1, 517, 4, 64, 128, 1, "bf16", 0, True),
    (2, 257, 6, 64, 64, 3, "bf16", 128, False),
    (1, 1, 2, 16, 32, 1, "f32", 0, True),
    (1, 1000, 2, 64, 128, 1, "f32", 256, True),
    (1, 150, 4, 16, 32, 4, "f32", 64, True),      # one head per group
    (1, 130, 16, 16, 256, 16, "bf16", 64, True),  # group sums too wide for the LDS slices: two-pass combine
]


def _ids(c):
    return "b{}_L{}_H{}_P{}_N{}_G{}_{}_Q{}_{}".format(*c[:8], "h0" if c[8] else "noh0")


def _grads(seed, case, dt_mode="config", with_D=True):
    b, L, H, P, N, G, dtype, chunk, full = case
    fi = make_forward_inputs(b, L, H, P, N, G, dtype, seed, dt_mode=dt_mode, with_D=with_D,
                             h0_std=0.4 if full else 0.0)
    rng = np.random.default_rng(seed + 7)
    from synth import round_to

    dy = round_to(rng.standard_normal(fi.x.shape), dtype)
    dfinal = round_to(rng.standard_normal((b, H, P, N)), "f32") if full else None
    ref = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, dy, dfinal)
    got = ssd_mod.backward(dev(fi.x, dtype), dev(fi.dt, dtype), dev(fi.A), dev(fi.B, dtype), dev(fi.C, dtype),
                           dev(fi.D), dev(fi.h0), dev(dy, dtype), dev(dfinal), chunk=chunk)
    torch.cuda.synchronize()
    return ref, {k: (None if v is None else host(v)) for k, v in got.items()}


def _check(ref, got, dtype, names=("dx", "ddt", "dB", "dC", "dA", "dD"), tol_dA=None):
    errs = {}
    for k in names:
        if ref[k] is None:
            continue
        tol = tol_dA if (k == "dA" and tol_dA is not None) else Y_TOL[dtype]
        assert np.all(np.isfinite(got[k])), f"{k}: non-finite values"
        e = rel_l2(got[k], ref[k])
        errs[k] = e
        assert e <= tol, f"{k}: rel L2 {e:.3e} > {tol:.0e}"
    errs["dh0"] = assert_close_state(got["dh0"], ref["dh0"], "dh0")
    print("rel L2 " + ", ".join(f"{k} {v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward(gpu_ssd, case):
    ref, got = _grads(300, case)
    _check(ref, got, case[6])


@pytest.mark.parametrize("mode", ["long_memory", "extreme", "zero"])
def test_backward_stress(gpu_ssd, mode):
    """Long memory (the adjoint crosses every chunk), huge steps (decay underflow), zero steps, fp32 io: every
    gradient at the fp32 bar.  The decay gradient is formed chunk by chunk from the chunk-start states (no
    long suffix sum of nearly cancelling terms), with the in-chunk decays taken from fp64 sums of the steps."""
    ref, got = _grads(301, (1, 700, 4, 32, 32, 1, "f32", 64, True), dt_mode=mode)
    _check(ref, got, "f32")


# bf16 io, headdim 64, dstate 64 or 128, chunk 64 or 128: the decay gradient is formed chunk by chunk and the
# transposed scans run in bf16 compute.  One chunk shorter than the chunk size, a length that is a whole
# number of chunks (no front padding of the reversed walks), chunk 64, groups, an odd number of heads per
# group, one head per group with 64 KB of combine slices, with and without h0 and dfinal.
LOCAL = [
    (1, 40, 2, 64, 64, 1, "bf16", 64, True),
    (2, 256, 4, 64, 128, 2, "bf16", 128, True),
    (1, 300, 2, 64, 128, 1, "bf16", 64, False),
    (2, 450, 6, 64, 64, 3, "bf16", 0, True),
    (1, 333, 3, 64, 128, 1, "bf16", 128, True),  # three heads per group: one head per workgroup, generic combine
    (1, 200, 8, 64, 128, 8, "bf16", 128, True),  # eight groups at dstate 128: the two-half combine's widest slices
]


@pytest.mark.parametrize("case", LOCAL, ids=_ids)
def test_backward_local(gpu_ssd, case):
    ref, got = _grads(305, case)
    _check(ref, got, "bf16")


@pytest.mark.parametrize("mode", ["long_memory", "extreme", "zero"])
def test_backward_local_stress(gpu_ssd, mode):
    """The chunk-local decay gradient under long memory, huge steps and zero steps (bf16 io)."""
    ref, got = _grads(306, (1, 700, 4, 64, 64, 1, "bf16", 128, True), dt_mode=mode)
    _check(ref, got, "bf16")


def test_backward_in_a_graph(gpu_ssd):
    """A backward call (the bf16 chunk-kernel path: some twenty launches on the caller's stream) captured in one
    graph replays to the oracle's gradients, replay after replay, with eager work between replays.  (Its LDS
    atomics add in no fixed order, so replays are compared with the oracle, not bit by bit.)"""
    case = (1, 517, 4, 64, 128, 1, "bf16", 0, True)
    b, L, H, P, N, G, dtype, chunk, _ = case
    fi = make_forward_inputs(b, L, H, P, N, G, dtype, 311, h0_std=0.4)
    rng = np.random.default_rng(318)
    from synth import round_to

    dy = round_to(rng.standard_normal(fi.x.shape), dtype)
    dfinal = round_to(rng.standard_normal((b, H, P, N)), "f32")
    ref = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, dy, dfinal)
    args = (dev(fi.x, dtype), dev(fi.dt, dtype), dev(fi.A), dev(fi.B, dtype), dev(fi.C, dtype), dev(fi.D),
            dev(fi.h0), dev(dy, dtype), dev(dfinal))
    nbytes = ssd_mod.backward_workspace_bytes(args[0], args[3])
    ws = torch.empty(nbytes, dtype=torch.uint8, device=args[0].device)
    eager = ssd_mod.backward(*args, workspace=ws)
    torch.cuda.synchronize()
    _check(ref, {k: (None if v is None else host(v)) for k, v in eager.items()}, "bf16")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = ssd_mod.backward(*args, workspace=ws)
    for rep in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _check(ref, {k: (None if v is None else host(v)) for k, v in out.items()}, "bf16")
        _ = (eager["dx"].float() * 2).sum().item()  # eager work between replays


def test_backward_without_D(gpu_ssd):
    ref, got = _grads(302, (2, 200, 4, 16, 32, 2, "f32", 64, True), with_D=False)
    assert got["dD"] is None
    _check(ref, got, "f32")


def test_backward_empty(gpu_ssd):
    """L = 0: dh0 = dfinal and zero parameter gradients."""
    fi = make_forward_inputs(2, 1, 2, 16, 16, 1, "f32", 303, h0_std=0.3)
    dfinal = np.random.default_rng(3).standard_normal((2, 2, 16, 16)).astype(np.float32).astype(np.float64)
    got = ssd_mod.backward(dev(fi.x[:, :0]), dev(fi.dt[:, :0]), dev(fi.A), dev(fi.B[:, :0]), dev(fi.C[:, :0]),
                           dev(fi.D), dev(fi.h0), dev(fi.x[:, :0]), dev(dfinal))
    torch.cuda.synchronize()
    assert np.array_equal(host(got["dh0"]), dfinal)
    assert np.all(host(got["dA"]) == 0) and np.all(host(got["dD"]) == 0)


def test_backward_workload_full(gpu_ssd):
    """The 2.7B-shaped workload (64K tokens, 80 heads) at full size: every gradient against the oracle over
    all heads, dB and dC (sums over the 80 heads of their group) included."""
    fi = make_config_inputs("cfg2_64k")
    rng = np.random.default_rng(304)
    from synth import round_to

    dy = round_to(rng.standard_normal(fi.x.shape), "bf16")
    b, L, H, P, N, G = fi.dims
    dfinal = round_to(rng.standard_normal((b, H, P, N)), "f32")
    got = ssd_mod.backward(dev(fi.x, "bf16"), dev(fi.dt, "bf16"), dev(fi.A), dev(fi.B, "bf16"), dev(fi.C, "bf16"),
                           dev(fi.D), None, dev(dy, "bf16"), dev(dfinal))
    torch.cuda.synchronize()
    got = {k: (None if v is None else host(v)) for k, v in got.items()}
    ref = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, None, dy, dfinal)
    _check(ref, got, "bf16")
