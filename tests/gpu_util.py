"""Helpers shared by the GPU parity tests: device transfer and the acceptance metrics."""

from __future__ import annotations

import numpy as np
import torch

#: relative L2 bound on y for fp32 and bf16 inputs; final-state max-abs bound as a fraction of its RMS
Y_TOL = {"f32": 1e-4, "bf16": 1e-2}
STATE_TOL = 1e-3

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(a, dtype: str = "f32"):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_TORCH[dtype]).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)


def state_err(got, ref) -> float:
    """max |got - ref| / RMS(ref) (0 when both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if rms == 0.0:
        return diff
    return diff / rms


def assert_close_y(got, ref, dtype: str, what: str = "y"):
    e = rel_l2(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert e <= Y_TOL[dtype], f"{what}: rel L2 {e:.3e} > {Y_TOL[dtype]:.0e}"
    return e


def assert_close_state(got, ref, what: str = "final state", tol: float = STATE_TOL):
    e = state_err(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: max abs err {e:.3e} x RMS > {tol:.0e}"
    return e
