"""Helpers shared by the GPU parity tests: device transfer and the acceptance metrics.

y is accepted on three levels, all of which must hold:

* global: relative L2 error over the whole output (the workload description's
  acceptance metric: 1e-4 for fp32 inputs, 1e-2 for bf16 inputs);
* per row: every row of outputs (the last axis: the P values of one
  (batch, token, head), or the channels of one token for the selective scan)
  satisfies ||d_row|| <= rel * ||ref_row|| + floor * rms_row, where rms_row is
  the root mean square of the reference row norms of the same head (the same
  index of the second-to-last axis);
* per element: |d| <= rel * |ref| + floor * rms, rms the larger of the same head's
  reference RMS and that of the element's own row (a row may sit far above its
  head's average, e.g. early tokens carrying a large initial state).

For bf16 outputs the relative parts start from 2^-8, the largest relative
error of rounding one value to bfloat16 (8 significant bits, nearest-even),
and add the kernels' own arithmetic error (bf16 operands rounded once each, ~2^-9
relative per term; measured ~1.1e-3 relative L2 over whole outputs once the
output rounding is taken out).  The floors cover outputs that are small next
to the terms that cancel in them.  A single wrong row or a wrong 16 x 16 tile,
which moves the global norm by less than its bound, fails the row check by a
wide margin (tests/test_parity_checks.py plants such mistakes on the CPU).
"""

from __future__ import annotations

import numpy as np
import torch

#: relative L2 bound on y for fp32 and bf16 inputs; final-state max-abs bound as a fraction of its RMS
Y_TOL = {"f32": 1e-4, "bf16": 1e-2}
STATE_TOL = 1e-3
#: per-row bound (relative part, floor as a fraction of the RMS row norm)
ROW_TOL = {"f32": (1e-4, 1e-5), "bf16": (2.0 ** -8 + 8e-3, 8e-3)}
#: per-element bound (relative part, floor as a fraction of the RMS of the reference)
ELEM_TOL = {"f32": (1e-4, 1e-4), "bf16": (2.0 ** -8 + 4e-3, 3e-2)}

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}
_BLOCK_ROWS = 1 << 20


def dev(a, dtype: str = "f32"):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_TORCH[dtype]).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def _rows(a) -> np.ndarray:
    a = np.asarray(a)
    if a.ndim == 0:
        return a.reshape(1, 1)
    return a.reshape(-1, a.shape[-1]) if a.shape[-1] else a.reshape(-1, 1)


def _grouped(a) -> np.ndarray:
    """View as (M, G, K): K = last axis (one row), G = the axis before it (heads; 1 if absent)."""
    a = np.asarray(a)
    if a.ndim < 2:
        return a.reshape(1, 1, -1)
    return a.reshape(-1, a.shape[-2], a.shape[-1])


def rel_l2(got, ref) -> float:
    g, r = _rows(got), _rows(ref)
    num = den = 0.0
    for i in range(0, g.shape[0], _BLOCK_ROWS):
        gb = g[i:i + _BLOCK_ROWS].astype(np.float64)
        rb = r[i:i + _BLOCK_ROWS].astype(np.float64)
        num += float(np.sum((gb - rb) ** 2))
        den += float(np.sum(rb ** 2))
    if den == 0.0:
        return float(np.sqrt(num))
    return float(np.sqrt(num / den))


def local_errors(got, ref, dtype: str):
    """Worst per-row and per-element error as a fraction of its bound (<= 1 passes), and where.

    The floors are taken per index of the second-to-last axis (per head for y laid out
    (..., H, P)), so a head whose outputs are all small is held to its own scale.
    Returns (row_ratio, flat_row_index, elem_ratio, flat_elem_index)."""
    g, r = _grouped(got), _grouped(ref)
    M, G, K = r.shape
    rrel, rfloor = ROW_TOL[dtype]
    erel, efloor = ELEM_TOL[dtype]
    blk = max(1, _BLOCK_ROWS // max(G, 1))
    sum_row2 = np.zeros(G)
    for i in range(0, M, blk):
        rb = r[i:i + blk].astype(np.float64)
        sum_row2 += np.sum(rb * rb, axis=(0, 2))
    rms_row = np.sqrt(sum_row2 / max(M, 1))          # (G,)
    rms_el = np.sqrt(sum_row2 / max(M * K, 1))       # (G,)
    worst_row = worst_el = 0.0
    at_row = at_el = -1
    for i in range(0, M, blk):
        gb = g[i:i + blk].astype(np.float64)
        rb = r[i:i + blk].astype(np.float64)
        d = gb - rb
        row_ratio = np.sqrt(np.sum(d * d, axis=2)) / (rrel * np.sqrt(np.sum(rb * rb, axis=2))
                                                      + rfloor * rms_row[None, :] + 1e-300)
        row_rms = np.sqrt(np.mean(rb * rb, axis=2))
        el_scale = np.maximum(rms_el[None, :], row_rms)[:, :, None]
        el_ratio = np.abs(d) / (erel * np.abs(rb) + efloor * el_scale + 1e-300)
        k = int(np.argmax(row_ratio))
        if row_ratio.flat[k] > worst_row or at_row < 0:
            worst_row, at_row = float(row_ratio.flat[k]), i * G + k
        k = int(np.argmax(el_ratio))
        if el_ratio.flat[k] > worst_el or at_el < 0:
            worst_el, at_el = float(el_ratio.flat[k]), i * G * K + k
    return worst_row, at_row, worst_el, at_el


def state_err(got, ref) -> float:
    """max |got - ref| / RMS(ref) (0 when both are zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    diff = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if rms == 0.0:
        return diff
    return diff / rms


def assert_close_y(got, ref, dtype: str, what: str = "y"):
    """Global relative L2, per-row and per-element bounds; returns the global relative L2."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    e = rel_l2(got, ref)
    assert e <= Y_TOL[dtype], f"{what}: rel L2 {e:.3e} > {Y_TOL[dtype]:.0e}"
    if got.size:
        wr, ir, we, ie = local_errors(got, ref, dtype)
        shape_rows = ref.shape[:-1] if ref.ndim > 1 else (1,)
        assert wr <= 1.0, (f"{what}: row {np.unravel_index(ir, shape_rows)} error is {wr:.2f}x its bound "
                           f"(global rel L2 {e:.3e})")
        assert we <= 1.0, (f"{what}: element {np.unravel_index(ie, ref.shape)} error is {we:.2f}x its bound "
                           f"(global rel L2 {e:.3e})")
        print(f"{what}: rel L2 {e:.3e}; worst row {wr:.3f}, worst element {we:.3f} of their bounds")
    return e


def assert_close_state(got, ref, what: str = "final state", tol: float = STATE_TOL):
    e = state_err(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: max abs err {e:.3e} x RMS > {tol:.0e}"
    return e
