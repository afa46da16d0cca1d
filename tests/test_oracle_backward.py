"""Pins of the fp64 backward oracle (ssd_oracle_backward) against the forward oracle.

The backward pass is the derivative of the forward's result, so its pins come from
the (separately pinned) forward oracle: central finite differences of the scalar
loss <dy, y> + <dfinal, final> along random directions, for every input, at sizes
that cross the oracle's 64-token recomputation blocks; a single-token closed form;
and linearity in the output gradients.  ``test_mutants_are_caught`` plants mistakes
in the backward's source and checks that some pin fails for each.
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
from synth import make_forward_inputs


def _inputs(seed, b=2, L=70, H=4, P=3, N=5, G=2, dt_mode="config"):
    fi = make_forward_inputs(b, L, H, P, N, G, "f32", seed, dt_mode=dt_mode, h0_std=0.5)
    rng = np.random.default_rng(seed + 1000)
    dy = rng.standard_normal(fi.x.shape)
    dfinal = rng.standard_normal((b, H, P, N))
    return fi, dy, dfinal


def _loss(fi, dy, dfinal, **over):
    args = dict(x=fi.x, dt=fi.dt, A=fi.A, B=fi.B, C=fi.C, D=fi.D, h0=fi.h0)
    args.update(over)
    r = oracle.forward(args["x"], args["dt"], args["A"], args["B"], args["C"], args["D"], args["h0"])
    return math.fsum((dy * r["y"]).ravel()) + math.fsum((dfinal * r["final"]).ravel())


def _fd_check(fi, dy, dfinal, grads, name, eps, tol, seed):
    base = getattr(fi, name)
    v = np.random.default_rng(seed).standard_normal(base.shape)
    if name == "dt":
        v = v * base  # keep the steps positive
    plus = _loss(fi, dy, dfinal, **{name: base + eps * v})
    minus = _loss(fi, dy, dfinal, **{name: base - eps * v})
    fd = (plus - minus) / (2 * eps)
    an = math.fsum((grads["d" + name] * v).ravel())
    assert abs(fd - an) <= tol * max(1.0, abs(fd)), f"d{name}: finite difference {fd:.12g} vs backward {an:.12g}"


GRADS = ["x", "dt", "A", "B", "C", "D", "h0"]


def pin_bwd_finite_differences():
    """Every gradient equals the central difference of the forward oracle's loss along a random
    direction (2 batch rows, 2 groups, 70 tokens: across a recomputation block boundary)."""
    fi, dy, dfinal = _inputs(1)
    g = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, dy, dfinal)
    for i, name in enumerate(GRADS):
        eps = 1e-5 if name in ("dt", "A") else 1e-3
        _fd_check(fi, dy, dfinal, g, name, eps, 1e-7, 50 + i)


def pin_bwd_finite_differences_long_memory():
    """Same, with long memory (the adjoint crosses many blocks) and no final-state gradient."""
    fi, dy, _ = _inputs(2, b=1, L=200, H=2, P=2, N=3, G=1, dt_mode="long_memory")
    zero = np.zeros((1, 2, 2, 3))
    g = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, dy, None)
    for i, name in enumerate(GRADS):
        eps = 1e-5 if name in ("dt", "A") else 1e-3
        _fd_check(fi, dy, zero, g, name, eps, 1e-7, 70 + i)


def pin_bwd_single_token():
    """L = 1, one head, P = N = 1: y = C (a h0 + dt x B) + D x, final = a h0 + dt x B, a = exp(dt A);
    the gradients written out by hand."""
    fi, _, _ = _inputs(3, b=1, L=1, H=1, P=1, N=1, G=1)
    x, d, A, B, C, D, h0 = (float(fi.x.ravel()[0]), float(fi.dt.ravel()[0]), float(fi.A[0]), float(fi.B.ravel()[0]),
                            float(fi.C.ravel()[0]), float(fi.D[0]), float(fi.h0.ravel()[0]))
    gy, gf = 0.7, -1.3
    g = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, np.full((1, 1, 1, 1), gy),
                        np.full((1, 1, 1, 1), gf))
    a = math.exp(d * A)
    s = a * h0 + d * x * B
    adj = gy * C + gf  # gradient w.r.t. the state after the token
    ref = {
        "dx": adj * d * B + gy * D,
        "ddt": adj * (x * B + A * a * h0),
        "dA": adj * d * a * h0,
        "dB": adj * d * x,
        "dC": gy * s,
        "dD": gy * x,
        "dh0": adj * a,
    }
    for k, v in ref.items():
        assert abs(float(np.asarray(g[k]).ravel()[0]) - v) < 1e-14 * max(1.0, abs(v)), k


def pin_bwd_linear_in_output_gradients():
    """The gradients are linear in (dy, dfinal) jointly."""
    fi, dy1, df1 = _inputs(4, L=30)
    _, dy2, df2 = _inputs(5, L=30)
    g1 = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, dy1, df1)
    g2 = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, dy2, df2)
    g3 = oracle.backward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, 2 * dy1 - dy2, 2 * df1 - df2)
    for k in g1:
        ref = 2 * g1[k] - g2[k]
        assert np.allclose(g3[k], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max()), k


PINS = [pin_bwd_finite_differences, pin_bwd_finite_differences_long_memory, pin_bwd_single_token,
        pin_bwd_linear_in_output_gradients]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_empty_sequence():
    """L = 0: dh0 = dfinal and every other gradient is empty or zero."""
    fi, dy, dfinal = _inputs(6, L=1)
    g = oracle.backward(fi.x[:, :0], fi.dt[:, :0], fi.A, fi.B[:, :0], fi.C[:, :0], fi.D, fi.h0, dy[:, :0], dfinal)
    assert np.array_equal(g["dh0"], dfinal)
    assert np.all(g["dA"] == 0) and np.all(g["dD"] == 0) and g["dx"].shape[1] == 0


MUTANTS = {
    "bwd_ddt_without_decay_term": ("ddt[bt * H + h] = dd + A[h] * a * gs;", "ddt[bt * H + h] = dd;"),
    "bwd_dx_without_dt": ("dx[(bt * H + h) * P + p] = d * gb +", "dx[(bt * H + h) * P + p] = gb +"),
    "bwd_dx_without_D": ("= d * gb + (D ? D[h] * dyt[p] : 0.0);", "= d * gb;"),
    "bwd_dB_without_dt": ("dBt[n] = d * sb;", "dBt[n] = sb;"),
    "bwd_dC_previous_state": ("sc += Scur[p * N + n] * dyt[p];", "sc += Sprev[p * N + n] * dyt[p];"),
    "bwd_no_adjoint_decay": ("for (int64_t e = 0; e < PN; ++e) Gs[e] *= a;", ""),
    "bwd_dA_without_dt": ("dAacc += d * a * gs;", "dAacc += a * gs;"),
    "bwd_dD_dropped": ("dDacc += dyt[p] * xt[p];", ""),
    "bwd_dfinal_ignored": ("Gs[e] = dfinal ? dfinal[bh * PN + e] : 0.0;", "Gs[e] = 0.0;"),
    "bwd_group_sum": ("for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {", "for (int64_t h = 0; h < hpg; ++h) {"),
    "bwd_wrong_checkpoint": ("memcpy(blk, ck + k * PN, sizeof(double) * PN);",
                             "memcpy(blk, ck + (k > 0 ? k - 1 : 0) * PN, sizeof(double) * PN);"),
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
