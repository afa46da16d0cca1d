"""Pins of the fp64 Mamba-1 selective-scan oracle against results fixed by the mathematics.

The selective scan of "3.3 Hardware-Aware algorithms and GPU memory hierarchy
optimisation" (section 2.1: abar = exp(delta A), zero-order-hold bbar; sections
3 and 4: the first-order recurrence and its output through C) is checked
against closed forms, a textbook convolution, brute force over the materialised
state, an ODE solver and invariants.  ``test_mutants_are_caught`` plants
plausible mistakes in the oracle source and checks that some pin fails for each.
"""

from __future__ import annotations

import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from synth import make_selective_inputs

TIGHT = 1e-12


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b.ravel()), 1e-300)
    return float(np.linalg.norm((a - b).ravel()) / den)


def _small(seed=0, b=2, L=29, Dc=6, N=5, G=2, h0=True, dt_mode="config"):
    return make_selective_inputs(b, L, Dc, N, G, "f32", seed, dt_mode=dt_mode, h0_std=0.5 if h0 else 0.0)


def _run(si, zoh=True, **kw):
    return oracle.selective_scan(si.x, si.delta, si.A, si.B, si.C, si.D, si.h0, zoh=zoh, **kw)


def _bbar_factor(dl, a, zoh):
    """Input factor of one (step, A) pair written from its definition (math library calls)."""
    if zoh and a != 0.0:
        return math.expm1(dl * a) / a
    return dl


def pin_sel_reduces_to_ssd():
    """With A[d, n] the same for every n the selective scan is the SSD recurrence with headdim 1:
    delta is the head step, x gains a unit headdim, and the ZOH factor is the SSD input step."""
    si = _small(seed=1)
    b, L, Dc, N, G = si.dims
    a_d = si.A[:, 0].copy()
    si.A = np.repeat(a_d[:, None], N, axis=1)
    x4 = si.x[..., None]
    h04 = si.h0[:, :, None, :]
    for zoh in (False, True):
        r = _run(si, zoh=zoh)
        dt_in = oracle.dt_frontend(si.delta, a_d, zoh=True)[1] if zoh else None
        ref = oracle.forward(x4, si.delta, a_d, si.B, si.C, si.D, h04, dt_in=dt_in)
        assert _rel(r["y"], ref["y"][..., 0]) < TIGHT
        assert _rel(r["final"], ref["final"][:, :, 0, :]) < TIGHT


def pin_sel_geometric_series():
    """Constant delta, x and B with h0 = 0: h_T[n] = bbar_n x (1 - a_n^T) / (1 - a_n), a_n distinct."""
    si = _small(seed=2, b=1, L=40, Dc=3, N=4, G=1, h0=False)
    L = si.x.shape[1]
    si.delta[:] = si.delta[:, :1, :]
    si.x[:] = si.x[:, :1, :]
    si.B[:] = si.B[:, :1]
    for zoh in (False, True):
        r = _run(si, zoh=zoh)
        for d in range(3):
            dl, xv = si.delta[0, 0, d], si.x[0, 0, d]
            hT = np.zeros(4)
            for n in range(4):
                a = math.exp(dl * si.A[d, n])
                hT[n] = _bbar_factor(dl, si.A[d, n], zoh) * si.B[0, 0, 0, n] * xv * (1.0 - a ** L) / (1.0 - a)
            assert _rel(r["final"][0, d], hT) < 1e-11
            y_last = float(np.dot(si.C[0, L - 1, 0], hT)) + si.D[d] * xv
            assert abs(r["y"][0, L - 1, d] - y_last) < 1e-11 * max(1.0, abs(y_last))


def pin_sel_lti_convolution():
    """delta, A, B, C constant in t and h0 = 0: y = x * K + D x with K_k = sum_n C_n a_n^k bbar_n,
    checked against numpy.convolve."""
    si = _small(seed=3, b=1, L=64, Dc=2, N=6, G=1, h0=False)
    L = si.x.shape[1]
    si.delta[:] = si.delta[:, :1, :]
    si.B[:] = si.B[:, :1]
    si.C[:] = si.C[:, :1]
    r = _run(si, zoh=True)
    for d in range(2):
        dl = si.delta[0, 0, d]
        a = np.exp(dl * si.A[d])
        fac = np.array([_bbar_factor(dl, si.A[d, n], True) for n in range(6)])
        K = np.array([np.sum(si.C[0, 0, 0] * a ** k * fac * si.B[0, 0, 0]) for k in range(L)])
        ref = np.convolve(si.x[0, :, d], K)[:L] + si.D[d] * si.x[0, :, d]
        assert _rel(r["y"][0, :, d], ref) < 1e-11


def pin_sel_homogeneous():
    """x = 0: final[d, n] = exp(A[d, n] sum_t delta_t) h0[d, n] and
    y_t = sum_n C_t[n] exp(A[d, n] sum_{k<=t} delta_k) h0[d, n]."""
    si = _small(seed=4)
    si.x[:] = 0.0
    r = _run(si)
    b, L, Dc, N, G = si.dims
    for bb in range(b):
        for d in range(Dc):
            g = d // (Dc // G)
            tot = math.fsum(si.delta[bb, :, d])
            assert _rel(r["final"][bb, d], np.exp(si.A[d] * tot) * si.h0[bb, d]) < TIGHT
            for t in (0, L // 2, L - 1):
                s = math.fsum(si.delta[bb, :t + 1, d])
                ref = float(np.dot(si.C[bb, t, g], np.exp(si.A[d] * s) * si.h0[bb, d]))
                assert abs(r["y"][bb, t, d] - ref) < 1e-12 * max(1.0, abs(ref))


def pin_sel_materialized():
    """Brute force over the materialised (b, L, Dc, N) state tensor: every h_t written as
    exp(A sum_{k<=t} delta) h0 + sum_{s<=t} exp(A sum_{k=s+1..t} delta) bbar_s x_s, with each
    segment sum taken directly."""
    si = _small(seed=5, b=1, L=12, Dc=3, N=4, G=1)
    L = 12
    for zoh in (False, True):
        r = _run(si, zoh=zoh)
        for d in range(3):
            for t in range(L):
                h = np.exp(si.A[d] * np.sum(si.delta[0, :t + 1, d])) * si.h0[0, d]
                for s in range(t + 1):
                    dec = np.exp(si.A[d] * np.sum(si.delta[0, s + 1:t + 1, d]))
                    fac = np.array([_bbar_factor(si.delta[0, s, d], si.A[d, n], zoh) for n in range(4)])
                    h = h + dec * fac * si.B[0, s, 0] * si.x[0, s, d]
                y = float(np.dot(si.C[0, t, 0], h)) + si.D[d] * si.x[0, t, d]
                assert abs(r["y"][0, t, d] - y) < 1e-12 * max(1.0, abs(y))
                if t == L - 1:
                    assert _rel(r["final"][0, d], h) < TIGHT


def pin_sel_zoh_solves_the_ode():
    """Zero-order hold: over each step the state follows h' = A h + B x with x held constant, so
    integrating that ODE with a general-purpose solver over the step length gives the same state."""
    from scipy.integrate import solve_ivp

    si = _small(seed=6, b=1, L=6, Dc=1, N=3, G=1)
    si.delta[:] = np.array([0.3, 0.05, 1.2, 0.7, 0.01, 0.4])[None, :, None]
    r = _run(si, zoh=True)
    h = si.h0[0, 0].copy()
    for t in range(6):
        rhs = lambda _, v, t=t: si.A[0] * v + si.B[0, t, 0] * si.x[0, t, 0]
        h = solve_ivp(rhs, (0.0, si.delta[0, t, 0]), h, rtol=1e-12, atol=1e-14).y[:, -1]
        y = float(np.dot(si.C[0, t, 0], h)) + si.D[0] * si.x[0, t, 0]
        assert abs(r["y"][0, t, 0] - y) < 1e-9
    assert _rel(r["final"][0, 0], h) < 1e-9


def pin_sel_split_resume():
    """Associativity / carried initial state: scan(0:k) then scan(k:L, h0 = its final state) equals
    scan(0:L)."""
    si = _small(seed=7, L=41)
    full = _run(si)
    k = 17
    a = oracle.selective_scan(si.x[:, :k], si.delta[:, :k], si.A, si.B[:, :k], si.C[:, :k], si.D, si.h0)
    c = oracle.selective_scan(si.x[:, k:], si.delta[:, k:], si.A, si.B[:, k:], si.C[:, k:], si.D, a["final"])
    assert _rel(np.concatenate([a["y"], c["y"]], axis=1), full["y"]) < TIGHT
    assert _rel(c["final"], full["final"]) < TIGHT


def pin_sel_groups():
    """Channel d reads B and C of group d // (Dc / G): a G = 2 problem equals two G = 1 problems."""
    si = _small(seed=8, Dc=6, G=2)
    r = _run(si)
    for g in range(2):
        sl = slice(3 * g, 3 * g + 3)
        sub = oracle.selective_scan(si.x[:, :, sl], si.delta[:, :, sl], si.A[sl], si.B[:, :, g:g + 1],
                                    si.C[:, :, g:g + 1], si.D[sl], si.h0[:, sl])
        assert _rel(r["y"][:, :, sl], sub["y"]) < TIGHT
        assert _rel(r["final"][:, sl], sub["final"]) < TIGHT


def pin_sel_linearity():
    """(y, final) is linear in (x, h0) jointly for fixed delta, A, B, C, D."""
    s1, s2 = _small(seed=9), _small(seed=10)
    s2.delta, s2.A, s2.B, s2.C, s2.D = s1.delta, s1.A, s1.B, s1.C, s1.D
    r1, r2 = _run(s1), _run(s2)
    s3 = _small(seed=9)
    s3.x = 2.0 * s1.x - 0.5 * s2.x
    s3.h0 = 2.0 * s1.h0 - 0.5 * s2.h0
    r3 = _run(s3)
    assert _rel(r3["y"], 2.0 * r1["y"] - 0.5 * r2["y"]) < 1e-11
    assert _rel(r3["final"], 2.0 * r1["final"] - 0.5 * r2["final"]) < 1e-11


def pin_sel_zero_A_entry():
    """A[d, n] = 0: no decay, and the zero-order-hold factor takes its limit delta, so the entry
    accumulates h0 + sum_t delta_t B_t[n] x_t in both input forms."""
    si = _small(seed=11, b=1, L=20, Dc=2, N=3, G=1)
    si.A[1, 2] = 0.0
    for zoh in (False, True):
        r = _run(si, zoh=zoh)
        ref = si.h0[0, 1, 2] + math.fsum(si.delta[0, t, 1] * si.B[0, t, 0, 2] * si.x[0, t, 1] for t in range(20))
        assert abs(r["final"][0, 1, 2] - ref) < 1e-12
        assert np.all(np.isfinite(r["y"]))


def pin_sel_delta_zero():
    """delta = 0: the state never moves, y_t = C_t.h0 + D x_t."""
    si = _small(seed=12, dt_mode="zero")
    r = _run(si)
    assert np.array_equal(r["final"], si.h0)
    b, L, Dc, N, G = si.dims
    for d in range(Dc):
        g = d // (Dc // G)
        ref = np.einsum("bln,bn->bl", si.C[:, :, g], si.h0[:, d]) + si.D[d] * si.x[:, :, d]
        assert _rel(r["y"][:, :, d], ref) < TIGHT


PINS = [
    pin_sel_reduces_to_ssd, pin_sel_geometric_series, pin_sel_lti_convolution, pin_sel_homogeneous,
    pin_sel_materialized, pin_sel_zoh_solves_the_ode, pin_sel_split_resume, pin_sel_groups,
    pin_sel_linearity, pin_sel_zero_A_entry, pin_sel_delta_zero,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_empty_sequence():
    """L = 0 returns h0 as the final state and no output rows."""
    si = _small(seed=13, L=1)
    r = oracle.selective_scan(si.x[:, :0], si.delta[:, :0], si.A, si.B[:, :0], si.C[:, :0], si.D, si.h0)
    assert r["y"].shape[1] == 0
    assert np.array_equal(r["final"], si.h0)


MUTANTS = {
    "sel_decay_sign": ("double abar = exp(dl * Ad[n]);", "double abar = exp(-dl * Ad[n]);"),
    "sel_zoh_without_division": ("bbar = expm1(dl * Ad[n]) / Ad[n] * Bt[n];", "bbar = expm1(dl * Ad[n]) * Bt[n];"),
    "sel_zoh_without_guard": ("if (zoh && Ad[n] != 0.0) bbar", "if (zoh) bbar"),
    "sel_euler_without_delta": ("double bbar = dl * Bt[n];", "double bbar = Bt[n];"),
    "sel_C_in_input": ("double bbar = dl * Bt[n];", "double bbar = dl * Ct[n];"),
    "sel_output_before_update": (
        "h[n] = abar * h[n] + bbar * xv;\n                acc += Ct[n] * h[n];",
        "acc += Ct[n] * h[n];\n                h[n] = abar * h[n] + bbar * xv;",
    ),
    "sel_dropped_D": ("acc + (Dskip ? Dskip[d] * xv : 0.0)", "acc"),
    "sel_A_row_offset": ("const double* Ad = A + d * N;", "const double* Ad = A + d;"),
    "sel_wrong_group": ("g = d / cpg;", "g = d % G;"),
    "sel_h0_ignored": ("if (h0) memcpy(h, h0 + bd * N, sizeof(double) * N);", ""),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed to build mutants")
def test_mutants_are_caught(monkeypatch):
    with open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")) as f:
        original = f.read()
    survivors = []
    with tempfile.TemporaryDirectory() as tmp:
        for name, (old, new) in MUTANTS.items():
            assert original.count(old) == 1, f"mutation anchor for {name} not found once in the oracle source"
            src = os.path.join(tmp, f"{name}.c")
            lib = os.path.join(tmp, f"lib_{name}.so")
            with open(src, "w") as f:
                f.write(original.replace(old, new))
            subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", lib, src,
                            "-lm"], check=True)
            monkeypatch.setattr(oracle, "_LIB_PATH", lib)
            monkeypatch.setattr(oracle, "_lib", None)
            caught = False
            for pin in PINS:
                try:
                    pin()
                except (AssertionError, ValueError, IndexError):
                    caught = True
                    break
            if not caught:
                survivors.append(name)
            monkeypatch.setattr(oracle, "_lib", None)
    assert not survivors, f"planted mistakes not caught by any pin: {survivors}"
