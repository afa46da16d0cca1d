"""GPU parity of each C-ABI call and of the one-shot forward against the fp64 oracle.

Inputs come from the seeded generators; every intermediate fed to a single
staged call is produced by the oracle (never by the HIP path).  Sizes span
several tiles and a ragged tail.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from synth import make_forward_inputs
from tests.gpu_util import assert_close_state, assert_close_y, dev, host, rel_l2

pytestmark = pytest.mark.gpu

# (b, L, H, P, N, G, Q, dtype): ragged L, several tiles, both io dtypes, G > 1, P/N extremes
CASES = [
    (2, 600, 4, 64, 128, 2, 256, "bf16"),
    (1, 300, 2, 16, 16, 1, 64, "f32"),
    (1, 257, 3, 32, 48, 1, 128, "bf16"),
    (2, 130, 2, 64, 64, 1, 64, "f32"),
    (1, 97, 2, 128, 256, 1, 32, "bf16"),
    (1, 70, 1, 256, 64, 1, 16, "bf16"),
    (1, 200, 2, 16, 1024, 1, 48, "f32"),
    (1, 512, 2, 64, 32, 2, 512, "bf16"),
    # fast chunk kernels (bf16, P = 64, N in {64, 128, 256, 512}, Q a multiple of 64, up to 4096)
    (1, 3000, 4, 64, 128, 1, 1024, "bf16"),
    (2, 1100, 6, 64, 64, 3, 512, "bf16"),
    (1, 700, 3, 64, 128, 1, 192, "bf16"),
    (1, 5000, 2, 64, 64, 1, 4096, "bf16"),
    # one head per wavefront, four heads of a group per workgroup (dstate 64 / 128): two groups,
    # several head quads, ragged tails, one sub-chunk and many
    (2, 1500, 8, 64, 128, 2, 512, "bf16"),
    (1, 4100, 12, 64, 128, 1, 2048, "bf16"),
    (1, 777, 4, 64, 64, 1, 256, "bf16"),
    (3, 130, 8, 64, 64, 1, 64, "bf16"),
    # wide-state fast kernels (dstate 256 / 512, one head per workgroup, 128-column blocks)
    (1, 700, 2, 64, 256, 1, 192, "bf16"),
    (2, 450, 4, 64, 512, 2, 256, "bf16"),
    (1, 1300, 3, 64, 256, 3, 1024, "bf16"),
]


def _ids(c):
    return "b{}_L{}_H{}_P{}_N{}_G{}_Q{}_{}".format(*c)


def _inputs(case, seed, **kw):
    b, L, H, P, N, G, Q, dt = case
    return make_forward_inputs(b, L, H, P, N, G, dt, seed, **kw)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_chunk_cumsum(gpu_ssd, case):
    fi = _inputs(case, 100)
    Q = case[6]
    dtt_ref, cs_ref = oracle.chunk_cumsum(fi.dt, fi.A, Q)
    dtt, cs = gpu_ssd.chunk_cumsum(dev(fi.dt, fi.dtype), dev(fi.A), Q)
    torch.cuda.synchronize()
    assert np.array_equal(host(dtt), dtt_ref.astype(np.float32).astype(np.float64))
    assert rel_l2(host(cs), cs_ref) < 2e-6


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_chunk_state(gpu_ssd, case):
    fi = _inputs(case, 101)
    Q = case[6]
    dtt_ref, cs_ref = oracle.chunk_cumsum(fi.dt, fi.A, Q)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, None, chunk=Q, chunk_states=True)
    states = gpu_ssd.chunk_state(dev(fi.x, fi.dtype), dev(fi.B, fi.dtype), dev(dtt_ref), dev(cs_ref), Q)
    torch.cuda.synchronize()
    got = host(states)
    assert_close_state(got, ref["chunk_local"], "chunk-local states")
    if fi.dtype == "f32":
        assert rel_l2(got, ref["chunk_local"]) < 1e-5


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_state_passing(gpu_ssd, case):
    fi = _inputs(case, 102, h0_std=0.3)
    Q = case[6]
    _, cs_ref = oracle.chunk_cumsum(fi.dt, fi.A, Q)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, chunk=Q, chunk_states=True)
    local32 = ref["chunk_local"].astype(np.float32).astype(np.float64)
    start_ref, fin_ref = oracle.state_passing(local32, cs_ref, fi.h0)
    states = dev(local32)
    states, fin = gpu_ssd.state_passing(states, dev(cs_ref), dev(fi.h0), seqlen=fi.x.shape[1], chunk=Q)
    torch.cuda.synchronize()
    assert rel_l2(host(states), start_ref) < 1e-5
    assert rel_l2(host(fin), fin_ref) < 1e-5
    assert_close_state(host(fin), fin_ref)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_chunk_scan(gpu_ssd, case):
    fi = _inputs(case, 103, h0_std=0.3)
    Q = case[6]
    dtt_ref, cs_ref = oracle.chunk_cumsum(fi.dt, fi.A, Q)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, chunk=Q, chunk_states=True)
    start32 = ref["chunk_start"].astype(np.float32).astype(np.float64)
    y_ref = oracle.chunk_scan(fi.x, fi.dt, fi.A, fi.B, fi.C, start32, fi.D, chunk=Q)
    y = gpu_ssd.chunk_scan(dev(fi.x, fi.dtype), dev(fi.B, fi.dtype), dev(fi.C, fi.dtype), dev(dtt_ref),
                           dev(cs_ref), dev(start32), dev(fi.D), chunk=Q)
    torch.cuda.synchronize()
    assert_close_y(host(y), y_ref, fi.dtype)


def _run_forward(gpu_ssd, fi, chunk):
    y, fin = gpu_ssd.forward(dev(fi.x, fi.dtype), dev(fi.dt, fi.dtype), dev(fi.A), dev(fi.B, fi.dtype),
                             dev(fi.C, fi.dtype), dev(fi.D), dev(fi.h0), chunk=chunk)
    torch.cuda.synchronize()
    return host(y), host(fin)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_forward(gpu_ssd, case):
    fi = _inputs(case, 104, h0_std=0.3)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y, fin = _run_forward(gpu_ssd, fi, case[6])
    assert_close_y(y, ref["y"], fi.dtype)
    assert_close_state(fin, ref["final"])


@pytest.mark.parametrize("mode", ["long_memory", "extreme", "per_head_bias", "zero", "bursts"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_stress(gpu_ssd, mode, dtype):
    """Long memory (chunk passing matters), extreme decay (underflow), wide dt spread, dt = 0, and bursts
    of very large steps between ordinary ones (the chunk kernels switch their state-scale mode)."""
    a_mode = "minus_one" if mode == "long_memory" else "config"
    fi = make_forward_inputs(1, 1100, 4, 64, 128, 1, dtype, 105, dt_mode=mode, a_mode=a_mode, h0_std=0.5)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y, fin = _run_forward(gpu_ssd, fi, 256)
    assert_close_y(y, ref["y"], dtype)
    assert_close_state(fin, ref["final"])


def test_forward_without_D_and_h0(gpu_ssd):
    fi = make_forward_inputs(2, 333, 4, 64, 64, 2, "bf16", 106, with_D=False)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C)
    y, fin = _run_forward(gpu_ssd, fi, 128)
    assert_close_y(y, ref["y"], "bf16")
    assert_close_state(fin, ref["final"])


@pytest.mark.parametrize("Q", [64, 128, 192, 256, 512, 2624, 0])
def test_forward_chunk_independent(gpu_ssd, Q):
    """The result does not depend on the chunk size (Q = 0: the library's choice)."""
    fi = make_forward_inputs(1, 1500, 4, 64, 128, 1, "bf16", 107, dt_mode="long_memory", a_mode="minus_one",
                             h0_std=0.2)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y, fin = _run_forward(gpu_ssd, fi, Q)
    assert_close_y(y, ref["y"], "bf16")
    assert_close_state(fin, ref["final"])


def test_forward_split_resume(gpu_ssd):
    """forward(0:k) then forward(k:L, h0 = its final state) matches the oracle over 0:L, k mod Q != 0."""
    fi = make_forward_inputs(1, 1000, 4, 64, 128, 1, "bf16", 108, dt_mode="long_memory", a_mode="minus_one")
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D)
    k = 389
    args = lambda sl: (dev(fi.x[:, sl], "bf16"), dev(fi.dt[:, sl], "bf16"), dev(fi.A), dev(fi.B[:, sl], "bf16"),
                       dev(fi.C[:, sl], "bf16"), dev(fi.D))
    y1, f1 = gpu_ssd.forward(*args(slice(0, k)), None, chunk=256)
    y2, f2 = gpu_ssd.forward(*args(slice(k, None)), f1, chunk=256)
    torch.cuda.synchronize()
    assert_close_y(np.concatenate([host(y1), host(y2)], axis=1), ref["y"], "bf16")
    assert_close_state(host(f2), ref["final"])


def test_forward_empty(gpu_ssd):
    """L = 0 returns h0 as the final state; batch 0 is a no-op."""
    fi = make_forward_inputs(2, 1, 2, 16, 16, 1, "f32", 109, h0_std=1.0)
    x = dev(fi.x[:, :0])
    y, fin = gpu_ssd.forward(x, dev(fi.dt[:, :0]), dev(fi.A), dev(fi.B[:, :0]), dev(fi.C[:, :0]), dev(fi.D),
                             dev(fi.h0), chunk=64)
    torch.cuda.synchronize()
    assert y.shape[1] == 0
    assert np.array_equal(host(fin), fi.h0)
    y, fin = gpu_ssd.forward(x, dev(fi.dt[:, :0]), dev(fi.A), dev(fi.B[:, :0]), dev(fi.C[:, :0]), dev(fi.D),
                             None, chunk=64)
    torch.cuda.synchronize()
    assert np.all(host(fin) == 0.0)
    fb = make_forward_inputs(0, 16, 2, 16, 16, 1, "f32", 110)
    y, fin = gpu_ssd.forward(dev(fb.x), dev(fb.dt), dev(fb.A), dev(fb.B), dev(fb.C), chunk=64)
    torch.cuda.synchronize()
    assert y.numel() == 0 and fin.numel() == 0


def test_forward_nan_propagates(gpu_ssd):
    """A NaN in x reaches y and the final state (no hang, no masking); other heads and
    earlier chunks stay finite.  Inside its chunk it may reach rows of the same 32-token
    block that precede it (a masked zero times NaN is NaN in the MFMA)."""
    fi = make_forward_inputs(1, 300, 2, 16, 16, 1, "f32", 111)
    fi.x[0, 150, 1, 3] = np.nan
    y, fin = _run_forward(gpu_ssd, fi, 64)
    assert np.all(np.isfinite(y[0, :, 0])) and np.all(np.isfinite(fin[0, 0]))
    assert np.all(np.isfinite(y[0, :128, 1]))
    assert np.isnan(y[0, 150, 1]).any() and np.isnan(y[0, 299, 1]).any()
    assert np.isnan(fin[0, 1]).any()


def test_step_matches_forward(gpu_ssd):
    """L steps of ssd_step reproduce the oracle forward on the same tokens."""
    fi = make_forward_inputs(2, 40, 4, 64, 128, 2, "bf16", 112, h0_std=0.3)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    S = dev(fi.h0)
    ys = []
    for t in range(fi.x.shape[1]):
        ys.append(host(gpu_ssd.step(S, dev(fi.x[:, t], "bf16"), dev(fi.dt[:, t], "bf16"), dev(fi.A),
                                    dev(fi.B[:, t], "bf16"), dev(fi.C[:, t], "bf16"), dev(fi.D))))
    torch.cuda.synchronize()
    assert_close_y(np.stack(ys, axis=1), ref["y"], "bf16")
    assert_close_state(host(S), ref["final"])


# dstate 4 N4 with N4 a power of two up to 64 takes the lane kernel (whole rows per workgroup: 4096 / N,
# at most P); the others the LDS-staged one.  Headdims that are not a multiple of the rows per workgroup
# leave a partial last block (48 = 32 + 16 at N = 128, 80 = 64 + 16 at N = 64, 144 = 128 + 16 at N = 32),
# and 48 rows at N = 16 are fewer than one pass of 256 threads covers (64).
@pytest.mark.parametrize("P,N,dtype,G", [(16, 16, "f32", 1), (64, 48, "bf16", 1), (32, 512, "bf16", 1),
                                         (256, 1024, "f32", 1), (128, 256, "bf16", 1), (48, 128, "bf16", 1),
                                         (80, 64, "f32", 1), (112, 256, "bf16", 2), (48, 16, "f32", 2),
                                         (144, 32, "bf16", 2), (64, 32, "bf16", 1)])
def test_step_shapes(gpu_ssd, P, N, dtype, G):
    fi = make_forward_inputs(3, 3, 4 if G == 2 else 5, P, N, G, dtype, 113, h0_std=0.2)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    S = dev(fi.h0)
    ys = [host(gpu_ssd.step(S, dev(fi.x[:, t], dtype), dev(fi.dt[:, t], dtype), dev(fi.A), dev(fi.B[:, t], dtype),
                            dev(fi.C[:, t], dtype), dev(fi.D))) for t in range(3)]
    torch.cuda.synchronize()
    assert_close_y(np.stack(ys, axis=1), ref["y"], dtype)
    assert_close_state(host(S), ref["final"])


# shapes that take the fused forward (chunk = 0, bf16, headdim 64, dstate 64 to 512): ragged tails,
# several segments, G > 1, h0, long memory, sequences shorter than one 64-token chunk
FUSED = [
    (1, 1, 4, 64, 128, 1, "config"),
    (1, 37, 3, 64, 64, 1, "config"),
    (2, 700, 4, 64, 128, 2, "config"),
    (1, 4096 + 77, 6, 64, 128, 3, "long_memory"),
    (3, 1500, 8, 64, 64, 2, "long_memory"),
    (1, 9000, 2, 64, 128, 1, "extreme"),
    (1, 20000, 4, 64, 64, 1, "per_head_bias"),
    (1, 1000, 4, 64, 256, 1, "long_memory"),
    (2, 333, 2, 64, 512, 2, "config"),
    (1, 3000, 2, 64, 512, 1, "extreme"),
    (1, 6000, 4, 64, 128, 1, "bursts"),
    (2, 2500, 2, 64, 64, 1, "bursts"),
    (1, 3000, 2, 64, 256, 1, "bursts"),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "b{}_L{}_H{}_P{}_N{}_G{}_{}".format(*c))
def test_forward_fused(gpu_ssd, case):
    b, L, H, P, N, G, mode = case
    a_mode = "minus_one" if mode == "long_memory" else "config"
    fi = make_forward_inputs(b, L, H, P, N, G, "bf16", 114, dt_mode=mode, a_mode=a_mode, h0_std=0.4)
    cfg = gpu_ssd.query_config(b, L, H, P, N, G, 0, torch.bfloat16)
    assert cfg["chunks_per_segment"] > 1 or L <= 256  # the fused path is the one taken
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y, fin = _run_forward(gpu_ssd, fi, 0)
    assert_close_y(y, ref["y"], "bf16")
    assert_close_state(fin, ref["final"])


def test_forward_many_chunks(gpu_ssd):
    """20000 tokens at the workload's decay rates: dozens of chunks, most of them attenuated far below
    fp32 range by the sequence end; outputs and final state stay within the tolerances."""
    fi = make_forward_inputs(1, 20000, 4, 64, 128, 1, "bf16", 131, h0_std=0.3)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y, fin = _run_forward(gpu_ssd, fi, 640)  # 32 chunks, the last one ragged
    assert_close_y(y, ref["y"], "bf16")
    assert_close_state(fin, ref["final"])


def test_forward_final_state_made_of_old_chunks(gpu_ssd):
    """x = 0 over the last 2000 tokens: the final state is only the older chunks' states, attenuated
    by about 2^-62 (A = -1, log-uniform steps); it still meets its bound relative to its own size,
    which any loss of precision in those older chunk states would break."""
    fi = make_forward_inputs(1, 4096, 4, 64, 128, 1, "bf16", 132, a_mode="minus_one", h0_std=0.3)
    fi.x[:, -2000:] = 0.0
    decay_log2 = -(fi.dt[0, -2000:, :].astype(np.float64).sum(axis=0)) * np.log2(np.e)
    assert np.all(decay_log2 < -40) and np.all(decay_log2 > -100)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y, fin = _run_forward(gpu_ssd, fi, 0)
    assert_close_y(y, ref["y"], "bf16")
    assert_close_state(fin, ref["final"])


@pytest.mark.parametrize("Q", [192, 2624])
def test_forward_non_power_of_two_chunks(gpu_ssd, Q):
    """Chunk sizes the library's rule picks (multiples of 64 that are not powers of two) over several
    chunks and a ragged tail (6000 = 2 x 2624 + 752), with long memory so the state pass matters."""
    fi = make_forward_inputs(1, 6000, 4, 64, 128, 1, "bf16", 133, dt_mode="long_memory", a_mode="minus_one",
                             h0_std=0.2)
    ref = oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y, fin = _run_forward(gpu_ssd, fi, Q)
    assert_close_y(y, ref["y"], "bf16")
    assert_close_state(fin, ref["final"])
