"""Seeded input generators for the Mamba-2 SSD forward scan, its decode step and the
Mamba-1 selective scan.

Value distributions follow the workload description of the SSD benchmark
configurations (tiny fp32 case, 130M-shaped, 2.7B-shaped, long-context state
sweep, decode step):

* x ~ N(0, 1)
* dt = softplus(z + b) with z ~ N(0, 1) and the bias b drawn per element so that
  dt is log-uniform on [1e-3, 0.1]: u ~ LogU[1e-3, 0.1], b = log(expm1(u)) - z.
  (A per-head bias cannot keep every element inside the interval; that variant
  is kept as the ``per_head_bias`` stress mode.)
* A_h = -exp(U(log 1, log 16))
* B, C ~ N(0, 1) / sqrt(N)
* D ~ N(0, 1)
* h0 = 0 for the prefill configurations; the decode state ~ N(0, 0.1^2)

The Mamba-1 selective scan takes the same recipes per channel: x ~ N(0, 1), the
step delta log-uniform on [1e-3, 0.1] (through the same softplus construction),
B, C ~ N(0, 1) / sqrt(N), D ~ N(0, 1), and A[d, n] = -exp(U(log 1, log 16))
drawn independently for every (channel, state) entry.

Everything is drawn in float64 from ``numpy.random.default_rng(seed)`` (PCG64)
and then rounded (round-to-nearest-even) to the storage dtype of the device
path: bfloat16 for x, dt, B, C in the bf16 configurations, float32 for A, D,
h0 and for everything in the fp32 configuration.  The returned arrays are
float64 copies of the rounded values, so the oracle sees exactly the numbers
the GPU sees.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

# ---------------------------------------------------------------------------
# rounding to device storage types (input preparation, not method arithmetic)
# ---------------------------------------------------------------------------


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float32 holding bf16 values."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    bits = f.view(np.uint32)
    # finite inputs cannot overflow 32 bits here: 0xFF7FFFFF + 0x8000 < 2**32
    rounded = (bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    out = rounded.view(np.float32)
    # keep non-finite values as they are (never produced by the generators)
    bad = ~np.isfinite(f)
    if bad.any():
        out = out.copy()
        out[bad] = f[bad]
    return out.reshape(np.shape(a))


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype and widen back to float64."""
    if dtype == "bf16":
        return bf16_round(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# workload shapes
# ---------------------------------------------------------------------------

K = 1024

#: The five benchmark workloads; every one is a synthetic, seeded problem.
CONFIGS: Dict[str, dict] = {
    # tiny fp32 forward
    "cfg0": dict(batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, ngroups=1, chunk=64, dtype="f32"),
    # Mamba-2-130M shaped forward
    "cfg1": dict(batch=4, seqlen=2 * K, nheads=24, headdim=64, dstate=128, ngroups=1, chunk=256, dtype="bf16"),
    # Mamba-2-2.7B shaped forward, L in {1K, 4K, 16K, 64K}
    "cfg2_1k": dict(batch=1, seqlen=1 * K, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=256, dtype="bf16"),
    "cfg2_4k": dict(batch=1, seqlen=4 * K, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=256, dtype="bf16"),
    "cfg2_16k": dict(batch=1, seqlen=16 * K, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=256, dtype="bf16"),
    "cfg2_64k": dict(batch=1, seqlen=64 * K, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=256, dtype="bf16"),
    # decode step on the 2.7B shape: 64 consecutive single-token updates
    "cfg4": dict(batch=64, seqlen=1, nheads=80, headdim=64, dstate=128, ngroups=1, chunk=0, dtype="bf16", steps=64),
}
# long-context state-size sweep, L in {64K, 256K} x N in {64, 128, 256, 512}
for _L in (64, 256):
    for _N in (64, 128, 256, 512):
        CONFIGS[f"cfg3_{_L}k_n{_N}"] = dict(
            batch=1, seqlen=_L * K, nheads=32, headdim=64, dstate=_N, ngroups=1, chunk=256, dtype="bf16"
        )


def config_shapes(name: str) -> dict:
    return dict(CONFIGS[name])


def seed_for(name: str) -> int:
    """Seed = configuration index; sweep points add 1000*index + 10*log2(L) + log2(N)."""
    cfg = CONFIGS[name]
    idx = int(name[3])
    if name in ("cfg0", "cfg1", "cfg4"):
        return idx
    return idx * 1000 + 10 * int(math.log2(cfg["seqlen"])) + int(math.log2(cfg["dstate"]))


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class ForwardInputs:
    x: np.ndarray  # (b, L, H, P)
    dt: np.ndarray  # (b, L, H)
    A: np.ndarray  # (H,)
    B: np.ndarray  # (b, L, G, N)
    C: np.ndarray  # (b, L, G, N)
    D: Optional[np.ndarray]  # (H,) or None
    h0: Optional[np.ndarray]  # (b, H, P, N) or None
    dtype: str  # storage dtype of x, dt, B, C (and y)

    @property
    def dims(self):
        b, L, H, P = self.x.shape
        G, N = self.B.shape[2], self.B.shape[3]
        return b, L, H, P, N, G


def _draw_dt(rng: np.random.Generator, shape, mode: str, nheads: int) -> np.ndarray:
    if mode == "config":
        # per-element bias: dt = softplus(z + log(expm1(u)) - z) = u, u log-uniform
        u = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), size=shape))
        z = rng.standard_normal(shape)
        bias = np.log(np.expm1(u)) - z
        return np.logaddexp(0.0, z + bias)
    if mode == "per_head_bias":
        # bias drawn once per head: dt spreads well outside [1e-3, 0.1]
        u = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), size=(nheads,)))
        z = rng.standard_normal(shape)
        return np.logaddexp(0.0, z + np.log(np.expm1(u)))
    if mode == "long_memory":
        # tiny steps: a 256-token chunk keeps about 90% of its state when A = -1
        return np.exp(rng.uniform(math.log(1e-4), math.log(1e-3), size=shape))
    if mode == "extreme":
        # very large steps: per-token decay down to exp(-32), exercising underflow
        return np.exp(rng.uniform(math.log(1e-3), math.log(2.0), size=shape))
    if mode == "zero":
        return np.zeros(shape)
    if mode == "bursts":
        # the workload's steps with bursts of very large ones (0.5 to 2, 20 to 90 tokens long, at
        # random offsets along the sequence axis), so that slowly and very quickly decaying stretches
        # alternate within one sequence
        dt = _draw_dt(rng, shape, "config", nheads)
        L = shape[1]
        flat = dt.reshape(shape[0], L, -1)
        for bi in range(shape[0]):
            for c in range(flat.shape[2]):
                t = int(rng.integers(0, 64))
                while t < L:
                    n = int(rng.integers(20, 91))
                    flat[bi, t:t + n, c] = rng.uniform(0.5, 2.0, size=min(n, L - t))
                    t += n + int(rng.integers(30, 400))
        return flat.reshape(shape)
    raise ValueError(f"unknown dt mode {mode!r}")


def make_forward_inputs(
    batch: int,
    seqlen: int,
    nheads: int,
    headdim: int,
    dstate: int,
    ngroups: int = 1,
    dtype: str = "bf16",
    seed: int = 0,
    *,
    dt_mode: str = "config",
    a_mode: str = "config",
    with_D: bool = True,
    h0_std: float = 0.0,
) -> ForwardInputs:
    """Draw one forward problem.  ``h0_std > 0`` adds an initial state ~ N(0, h0_std^2)."""
    if nheads % ngroups:
        raise ValueError("nheads must be a multiple of ngroups")
    rng = np.random.default_rng(seed)
    b, L, H, P, N, G = batch, seqlen, nheads, headdim, dstate, ngroups
    x = rng.standard_normal((b, L, H, P))
    dt = _draw_dt(rng, (b, L, H), dt_mode, H)
    if a_mode == "config":
        A = -np.exp(rng.uniform(0.0, math.log(16.0), size=(H,)))
    elif a_mode == "minus_one":
        A = -np.ones(H)
    else:
        raise ValueError(f"unknown A mode {a_mode!r}")
    Bm = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    Cm = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    D = rng.standard_normal((H,)) if with_D else None
    h0 = rng.standard_normal((b, H, P, N)) * h0_std if h0_std > 0 else None
    return ForwardInputs(
        x=round_to(x, dtype),
        dt=round_to(dt, dtype),
        A=round_to(A, "f32"),
        B=round_to(Bm, dtype),
        C=round_to(Cm, dtype),
        D=None if D is None else round_to(D, "f32"),
        h0=None if h0 is None else round_to(h0, "f32"),
        dtype=dtype,
    )


def make_config_inputs(name: str, seed: Optional[int] = None, **overrides) -> ForwardInputs:
    cfg = CONFIGS[name]
    return make_forward_inputs(
        cfg["batch"], cfg["seqlen"], cfg["nheads"], cfg["headdim"], cfg["dstate"], cfg["ngroups"],
        cfg["dtype"], seed_for(name) if seed is None else seed, **overrides,
    )


@dataclasses.dataclass
class StepInputs:
    state0: np.ndarray  # (b, H, P, N) float32 values
    A: np.ndarray  # (H,)
    D: Optional[np.ndarray]  # (H,)
    x: np.ndarray  # (steps, b, H, P)
    dt: np.ndarray  # (steps, b, H)
    B: np.ndarray  # (steps, b, G, N)
    C: np.ndarray  # (steps, b, G, N)
    dtype: str


def make_step_inputs(
    batch: int,
    nheads: int,
    headdim: int,
    dstate: int,
    ngroups: int = 1,
    steps: int = 64,
    dtype: str = "bf16",
    seed: int = 4,
    state_std: float = 0.1,
    with_D: bool = True,
) -> StepInputs:
    """Decode workload: A, D and the state drawn once, then fresh x, dt, B, C per step."""
    rng = np.random.default_rng(seed)
    b, H, P, N, G = batch, nheads, headdim, dstate, ngroups
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=(H,)))
    D = rng.standard_normal((H,)) if with_D else None
    state0 = rng.standard_normal((b, H, P, N)) * state_std
    xs, dts, Bs, Cs = [], [], [], []
    for _ in range(steps):
        xs.append(rng.standard_normal((b, H, P)))
        dts.append(_draw_dt(rng, (b, H), "config", H))
        Bs.append(rng.standard_normal((b, G, N)) / math.sqrt(N))
        Cs.append(rng.standard_normal((b, G, N)) / math.sqrt(N))
    return StepInputs(
        state0=round_to(state0, "f32"),
        A=round_to(A, "f32"),
        D=None if D is None else round_to(D, "f32"),
        x=round_to(np.stack(xs), dtype),
        dt=round_to(np.stack(dts), dtype),
        B=round_to(np.stack(Bs), dtype),
        C=round_to(np.stack(Cs), dtype),
        dtype=dtype,
    )


# ---------------------------------------------------------------------------
# Mamba-1 selective scan
# ---------------------------------------------------------------------------

#: Selective-scan workload: the 2.7B-shaped width (80 heads x 64 = 5120 channels) at the longest
#: 2.7B sequence length, with Mamba-1's per-channel diagonal state of 16 entries.
SELECTIVE_CONFIGS: Dict[str, dict] = {
    "mamba1_5120ch_64k": dict(batch=1, seqlen=64 * K, channels=5120, dstate=16, ngroups=1, dtype="bf16"),
}


@dataclasses.dataclass
class SelectiveInputs:
    x: np.ndarray  # (b, L, Dc)
    delta: np.ndarray  # (b, L, Dc): the step after the front-end
    A: np.ndarray  # (Dc, N)
    B: np.ndarray  # (b, L, G, N)
    C: np.ndarray  # (b, L, G, N)
    D: Optional[np.ndarray]  # (Dc,) or None
    h0: Optional[np.ndarray]  # (b, Dc, N) or None
    dtype: str

    @property
    def dims(self):
        b, L, Dc = self.x.shape
        G, N = self.B.shape[2], self.B.shape[3]
        return b, L, Dc, N, G


def make_selective_inputs(
    batch: int,
    seqlen: int,
    channels: int,
    dstate: int,
    ngroups: int = 1,
    dtype: str = "bf16",
    seed: int = 0,
    *,
    dt_mode: str = "config",
    with_D: bool = True,
    h0_std: float = 0.0,
) -> SelectiveInputs:
    """Draw one selective-scan problem (delta modes as for the SSD step)."""
    if channels % ngroups:
        raise ValueError("channels must be a multiple of ngroups")
    rng = np.random.default_rng(seed)
    b, L, Dc, N, G = batch, seqlen, channels, dstate, ngroups
    x = rng.standard_normal((b, L, Dc))
    delta = _draw_dt(rng, (b, L, Dc), dt_mode, Dc)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=(Dc, N)))
    Bm = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    Cm = rng.standard_normal((b, L, G, N)) / math.sqrt(N)
    D = rng.standard_normal((Dc,)) if with_D else None
    h0 = rng.standard_normal((b, Dc, N)) * h0_std if h0_std > 0 else None
    return SelectiveInputs(
        x=round_to(x, dtype),
        delta=round_to(delta, dtype),
        A=round_to(A, "f32"),
        B=round_to(Bm, dtype),
        C=round_to(Cm, dtype),
        D=None if D is None else round_to(D, "f32"),
        h0=None if h0 is None else round_to(h0, "f32"),
        dtype=dtype,
    )


def make_selective_config_inputs(name: str, seed: int = 5) -> SelectiveInputs:
    cfg = SELECTIVE_CONFIGS[name]
    return make_selective_inputs(cfg["batch"], cfg["seqlen"], cfg["channels"], cfg["dstate"], cfg["ngroups"],
                                 cfg["dtype"], seed)
