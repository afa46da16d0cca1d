"""Pins of the fp64 oracle against results fixed by the mathematics, not by itself.

Each ``pin_*`` function checks the C oracle (``oracle`` package) against a
closed form, a textbook routine, brute force on tiny inputs, or an invariant
of the recurrence.  ``test_mutants_are_caught`` recompiles the oracle with
plausible mistakes planted in its source and checks that some pin fails for
every one of them.
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
from oracle import ssd_ref
from synth import make_forward_inputs, make_step_inputs

LOG2E = 1.0 / math.log(2.0)
TIGHT = 1e-12


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.linalg.norm(b.ravel()), 1e-300)
    return float(np.linalg.norm((a - b).ravel()) / den)


def _small(seed=0, b=2, L=37, H=4, P=3, N=5, G=2, h0=True, dt_mode="config"):
    return make_forward_inputs(b, L, H, P, N, G, "f32", seed, dt_mode=dt_mode, h0_std=0.5 if h0 else 0.0)


def _fwd(fi, **kw):
    return oracle.forward(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, **kw)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------


def pin_decay_closed_form():
    """x = 0: the state only decays, final = exp(A sum dt) h0 and y_t = exp(A sum_{k<=t} dt) C_t.h0."""
    fi = _small(seed=1)
    fi.x[:] = 0.0
    r = _fwd(fi)
    b, L, H, P, N, G = fi.dims
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            tot = math.fsum(fi.dt[bb, :, h])
            assert _rel(r["final"][bb, h], math.exp(fi.A[h] * tot) * fi.h0[bb, h]) < TIGHT
            for t in (0, L // 2, L - 1):
                part = math.fsum(fi.dt[bb, : t + 1, h])
                want = math.exp(fi.A[h] * part) * (fi.h0[bb, h] @ fi.C[bb, t, g])
                assert _rel(r["y"][bb, t, h], want) < TIGHT


def pin_geometric_series():
    """dt, x, B constant, h0 = 0: S_T = dt x (outer) B (1 - a^T) / (1 - a), a = exp(dt A)."""
    b, L, H, P, N, G = 1, 50, 3, 4, 6, 1
    rng = np.random.default_rng(7)
    x1 = rng.standard_normal((H, P))
    B1 = rng.standard_normal(N)
    d = np.array([0.01, 0.1, 0.7])
    A = np.array([-1.0, -3.0, -0.25])
    x = np.broadcast_to(x1, (b, L, H, P)).copy()
    dt = np.broadcast_to(d, (b, L, H)).copy()
    Bm = np.broadcast_to(B1, (b, L, G, N)).copy()
    Cm = rng.standard_normal((b, L, G, N))
    r = oracle.forward(x, dt, A, Bm, Cm)
    for h in range(H):
        a = math.exp(d[h] * A[h])
        want = d[h] * np.outer(x1[h], B1) * (1.0 - a ** L) / (1.0 - a)
        assert _rel(r["final"][0, h], want) < 1e-12


def pin_lti_convolution():
    """dt, A, B, C constant in t: y = causal convolution of x with K_k = dt (C.B) a^k, plus D x."""
    b, L, H, P, N, G = 1, 64, 2, 3, 4, 1
    rng = np.random.default_rng(11)
    x = rng.standard_normal((b, L, H, P))
    d = np.array([0.05, 0.3])
    A = np.array([-2.0, -0.5])
    B1 = rng.standard_normal(N)
    C1 = rng.standard_normal(N)
    D = np.array([0.7, -1.3])
    dt = np.broadcast_to(d, (b, L, H)).copy()
    Bm = np.broadcast_to(B1, (b, L, G, N)).copy()
    Cm = np.broadcast_to(C1, (b, L, G, N)).copy()
    r = oracle.forward(x, dt, A, Bm, Cm, D)
    for h in range(H):
        a = math.exp(d[h] * A[h])
        kern = d[h] * float(C1 @ B1) * a ** np.arange(L)
        for p in range(P):
            want = np.convolve(x[0, :, h, p], kern)[:L] + D[h] * x[0, :, h, p]
            assert _rel(r["y"][0, :, h, p], want) < 1e-12


def pin_single_token():
    """L = 1: y = C.(exp(dt A) h0 + dt x (outer) B) + D x."""
    fi = _small(seed=3, L=1)
    r = _fwd(fi)
    b, L, H, P, N, G = fi.dims
    for bb in range(b):
        for h in range(H):
            g = h // (H // G)
            d = fi.dt[bb, 0, h]
            S = math.exp(d * fi.A[h]) * fi.h0[bb, h] + d * np.outer(fi.x[bb, 0, h], fi.B[bb, 0, g])
            assert _rel(r["final"][bb, h], S) < TIGHT
            assert _rel(r["y"][bb, 0, h], S @ fi.C[bb, 0, g] + fi.D[h] * fi.x[bb, 0, h]) < TIGHT


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------


def pin_materialized_and_quadratic():
    """Recurrence == every state written out == the quadratic (semiseparable) form."""
    fi = _small(seed=5, L=29)
    r = _fwd(fi)
    y_m, fin_m, _ = ssd_ref.materialized(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    y_q = ssd_ref.quadratic(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0)
    assert _rel(r["y"], y_m) < TIGHT
    assert _rel(r["final"], fin_m) < TIGHT
    assert _rel(r["y"], y_q) < TIGHT


def pin_chunk_decomposition():
    """The fp64 chunked form equals the recurrence for every chunk size (Q = 1 .. L)."""
    fi = _small(seed=6, L=64)
    r = _fwd(fi)
    for Q in (1, 2, 3, 16, 64, 5, 100):
        c = ssd_ref.chunked(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, Q=Q)
        assert _rel(c["y"], r["y"]) < 1e-11, Q
        assert _rel(c["final"], r["final"]) < 1e-11, Q


def pin_staged_calls():
    """Each staged oracle call equals the intermediate of the fp64 chunked form."""
    fi = _small(seed=8, L=45)
    Q = 8
    c = ssd_ref.chunked(fi.x, fi.dt, fi.A, fi.B, fi.C, fi.D, fi.h0, Q=Q)
    r = _fwd(fi, chunk=Q, chunk_states=True)
    dtt, cs = oracle.chunk_cumsum(fi.dt, fi.A, Q)
    assert _rel(cs, c["cs_log2"]) < 1e-13
    b, L, H = fi.dt.shape
    pad = np.zeros((b, cs.shape[2] * Q, H))
    pad[:, :L] = fi.dt
    assert np.array_equal(dtt, pad.reshape(b, -1, Q, H).transpose(0, 3, 1, 2))
    assert _rel(r["chunk_local"], c["chunk_local"]) < 1e-11
    assert _rel(r["chunk_start"], c["chunk_start"]) < 1e-11
    start, fin = oracle.state_passing(r["chunk_local"], cs, fi.h0)
    assert _rel(start, c["chunk_start"]) < 1e-11
    assert _rel(fin, r["final"]) < 1e-11
    y = oracle.chunk_scan(fi.x, fi.dt, fi.A, fi.B, fi.C, r["chunk_start"], fi.D, chunk=Q)
    assert _rel(y, r["y"]) < 1e-12


def pin_cumsum_worked_example():
    """A hand-computed chunk cumulative sum in log2 units, with a zero-padded ragged tail.

    dt = (0.1, 0.2, 0.3, 0.4, 0.5), A = -2, Q = 2: the chunk sums of dt*A are
    (-0.2, -0.6), (-0.6, -1.4), (-1.0, -1.0) (the last position is padding).
    """
    dt = np.array([0.1, 0.2, 0.3, 0.4, 0.5]).reshape(1, 5, 1)
    dtt, cs = oracle.chunk_cumsum(dt, np.array([-2.0]), 2)
    want = np.array([[-0.2, -0.6], [-0.6, -1.4], [-1.0, -1.0]]) * LOG2E
    assert np.allclose(cs[0, 0], want, rtol=1e-14, atol=0)
    assert np.array_equal(dtt[0, 0], np.array([[0.1, 0.2], [0.3, 0.4], [0.5, 0.0]]))


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------


def pin_dt_zero():
    """dt = 0 leaves the state unchanged and gives y = C.h0 + D x (= D x when h0 = 0)."""
    fi = _small(seed=9, dt_mode="zero")
    r = _fwd(fi)
    assert _rel(r["final"], fi.h0) < TIGHT
    b, L, H, P, N, G = fi.dims
    for h in range(H):
        g = h // (H // G)
        want = np.einsum("btn,bpn->btp", fi.C[:, :, g], fi.h0[:, h]) + fi.D[h] * fi.x[:, :, h]
        assert _rel(r["y"][:, :, h], want) < TIGHT
    fi0 = _small(seed=9, dt_mode="zero", h0=False)
    r0 = _fwd(fi0)
    assert np.all(r0["final"] == 0.0)
    assert _rel(r0["y"], fi0.D[None, None, :, None] * fi0.x) < TIGHT


def pin_split_resume():
    """forward(0:k) then forward(k:L, h0 = its final state) == forward(0:L)."""
    fi = _small(seed=10, L=61)
    full = _fwd(fi)
    for k in (1, 13, 32, 60):
        a = oracle.forward(fi.x[:, :k], fi.dt[:, :k], fi.A, fi.B[:, :k], fi.C[:, :k], fi.D, fi.h0)
        bb = oracle.forward(fi.x[:, k:], fi.dt[:, k:], fi.A, fi.B[:, k:], fi.C[:, k:], fi.D, a["final"])
        assert _rel(np.concatenate([a["y"], bb["y"]], axis=1), full["y"]) < TIGHT
        assert _rel(bb["final"], full["final"]) < TIGHT


def pin_step_equals_forward():
    """L decode steps reproduce the forward pass on the same tokens."""
    fi = _small(seed=12, L=20)
    full = _fwd(fi)
    S = np.array(fi.h0, dtype=np.float64, copy=True)
    ys = []
    for t in range(fi.x.shape[1]):
        ys.append(oracle.step(S, fi.x[:, t], fi.dt[:, t], fi.A, fi.B[:, t], fi.C[:, t], fi.D))
    assert _rel(np.stack(ys, axis=1), full["y"]) < TIGHT
    assert _rel(S, full["final"]) < TIGHT


def pin_step_inputs_roundtrip():
    """The decode generator's per-step tensors drive the step recurrence consistently."""
    si = make_step_inputs(2, 3, 4, 5, 1, steps=6, dtype="bf16", seed=1)
    x = np.transpose(si.x, (1, 0, 2, 3))
    dt = np.transpose(si.dt, (1, 0, 2))
    B = np.transpose(si.B, (1, 0, 2, 3))
    C = np.transpose(si.C, (1, 0, 2, 3))
    full = oracle.forward(x, dt, si.A, B, C, si.D, si.state0)
    S = si.state0.copy()
    for t in range(6):
        y = oracle.step(S, si.x[t], si.dt[t], si.A, si.B[t], si.C[t], si.D)
        assert _rel(y, full["y"][:, t]) < TIGHT
    assert _rel(S, full["final"]) < TIGHT


def pin_linearity():
    """(y, final) is linear in (x, h0) jointly for fixed dt, A, B, C (with D)."""
    f1 = _small(seed=13)
    f2 = _small(seed=14)
    f2.dt[:] = f1.dt
    f2.B[:] = f1.B
    f2.C[:] = f1.C
    f2.A[:] = f1.A
    f2.D[:] = f1.D
    r1, r2 = _fwd(f1), _fwd(f2)
    al, be = 0.75, -2.5
    r3 = oracle.forward(al * f1.x + be * f2.x, f1.dt, f1.A, f1.B, f1.C, f1.D, al * f1.h0 + be * f2.h0)
    assert _rel(r3["y"], al * r1["y"] + be * r2["y"]) < 1e-12
    assert _rel(r3["final"], al * r1["final"] + be * r2["final"]) < 1e-12


def pin_head_permutation():
    """Heads are independent: permuting heads with A and D permutes the outputs (one group)."""
    fi = _small(seed=15, G=1)
    r = _fwd(fi)
    perm = np.array([2, 0, 3, 1])
    rp = oracle.forward(fi.x[:, :, perm], fi.dt[:, :, perm], fi.A[perm], fi.B, fi.C, fi.D[perm], fi.h0[:, perm])
    assert _rel(rp["y"], r["y"][:, :, perm]) < TIGHT
    assert _rel(rp["final"], r["final"][:, perm]) < TIGHT


def pin_groups():
    """With G groups, head h reads group h // (H/G): equals G separate one-group problems."""
    fi = _small(seed=16, H=6, G=3)
    r = _fwd(fi)
    for g in range(3):
        hs = slice(2 * g, 2 * g + 2)
        rg = oracle.forward(fi.x[:, :, hs], fi.dt[:, :, hs], fi.A[hs], fi.B[:, :, g:g + 1], fi.C[:, :, g:g + 1],
                            fi.D[hs], fi.h0[:, hs])
        assert _rel(rg["y"], r["y"][:, :, hs]) < TIGHT
        assert _rel(rg["final"], r["final"][:, hs]) < TIGHT


# ---------------------------------------------------------------------------
# dt front-end: bias + softplus + clamp, and the zero-order-hold input factor
# ---------------------------------------------------------------------------


def pin_frontend_softplus():
    """softplus(raw + bias) equals NumPy's logaddexp(0, .) (a library routine), including large
    positive and negative arguments; the clamp bounds it; without ZOH the input step is the step."""
    rng = np.random.default_rng(40)
    raw = np.concatenate([rng.normal(0.0, 3.0, (50, 4)), np.array([[-60.0, -20.0, 20.0, 60.0]])])
    bias = rng.normal(0.0, 1.0, 4)
    A = -np.exp(rng.uniform(0.0, math.log(16.0), 4))
    dec, inp = oracle.dt_frontend(raw, A, bias, softplus=True)
    want = np.logaddexp(0.0, raw + bias)
    assert np.max(np.abs(dec - want) / want) < 1e-14
    assert np.array_equal(inp, dec)
    dec_c, _ = oracle.dt_frontend(raw, A, bias, softplus=True, clamp=(1e-3, 0.1))
    assert dec_c.min() >= 1e-3 and dec_c.max() <= 0.1
    inside = (want > 1e-3) & (want < 0.1)
    assert inside.any() and np.array_equal(dec_c[inside], dec[inside])
    dec_n, _ = oracle.dt_frontend(raw, A)  # no bias, no softplus: the raw step itself
    assert np.array_equal(dec_n, raw)


def pin_zoh_factor_matrix_exponential():
    """The ZOH input factor is the top-right entry of expm([[A, 1], [0, 0]] d) (the augmented-matrix
    construction of a zero-order hold), computed by scipy.linalg.expm; small steps tend to d."""
    from scipy.linalg import expm

    rng = np.random.default_rng(41)
    d = np.exp(rng.uniform(math.log(1e-4), math.log(2.0), (6, 5)))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), 5))
    dec, inp = oracle.dt_frontend(d, A, zoh=True)
    assert np.array_equal(dec, d)
    for r in range(d.shape[0]):
        for h in range(d.shape[1]):
            m = expm(np.array([[A[h], 1.0], [0.0, 0.0]]) * d[r, h])
            assert abs(inp[r, h] - m[0, 1]) <= 1e-12 * abs(m[0, 1])
    tiny = np.full((1, 5), 1e-9)
    _, inp_t = oracle.dt_frontend(tiny, A, zoh=True)
    assert np.max(np.abs(inp_t / tiny - 1.0)) < 1e-7


def pin_zoh_forward_solves_the_ode():
    """With the ZOH input step the recurrence is the exact solution of S' = A S + B x with x, B held
    over each token's interval: one state (P = N = 1) integrated by scipy's solve_ivp."""
    from scipy.integrate import solve_ivp

    rng = np.random.default_rng(42)
    L = 12
    A = np.array([-3.0])
    d = np.exp(rng.uniform(math.log(1e-2), math.log(0.5), (1, L, 1)))
    x = rng.normal(size=(1, L, 1, 1))
    B = rng.normal(size=(1, L, 1, 1))
    C = rng.normal(size=(1, L, 1, 1))
    h0 = np.array([[[[0.7]]]])
    dec, inp = oracle.dt_frontend(d, A, zoh=True)
    r = oracle.forward(x, dec, A, B, C, None, h0, dt_in=inp)
    s = 0.7
    for t in range(L):
        sol = solve_ivp(lambda _, v: A[0] * v + B[0, t, 0, 0] * x[0, t, 0, 0], (0.0, d[0, t, 0]), [s],
                        rtol=1e-12, atol=1e-14)
        s = sol.y[0, -1]
        assert abs(r["y"][0, t, 0, 0] - C[0, t, 0, 0] * s) < 1e-9
    assert abs(r["final"][0, 0, 0, 0] - s) < 1e-9


def pin_input_step_only_scales_the_input():
    """A separate input step leaves the decay alone: with x = 0 the result ignores dt_in, and with
    h0 = 0 scaling dt_in by k scales y and the final state by k (linearity in the input term)."""
    fi = _small(seed=43)
    r1 = _fwd(fi)
    r2 = _fwd(fi, dt_in=fi.dt * 2.0)
    fi0 = _small(seed=43)
    fi0.x[:] = 0.0
    assert _rel(_fwd(fi0, dt_in=fi0.dt * 5.0)["final"], _fwd(fi0)["final"]) < TIGHT
    fih = _small(seed=43, h0=False)
    ra, rb = _fwd(fih), _fwd(fih, dt_in=fih.dt * 3.0)
    assert _rel(rb["final"], 3.0 * ra["final"]) < TIGHT
    d_x = (fih.D[None, None, :, None] * fih.x)
    assert _rel(rb["y"] - d_x, 3.0 * (ra["y"] - d_x)) < TIGHT
    assert _rel(r1["final"], r2["final"]) > 1e-3  # it does change the result
    dtt, cs = oracle.chunk_cumsum(fi.dt, fi.A, 16, dt_in=fi.dt * 2.0)
    dtt0, cs0 = oracle.chunk_cumsum(fi.dt, fi.A, 16)
    assert np.array_equal(cs, cs0) and np.array_equal(dtt, 2.0 * dtt0)


PINS = [
    pin_decay_closed_form, pin_geometric_series, pin_lti_convolution, pin_single_token,
    pin_materialized_and_quadratic, pin_chunk_decomposition, pin_staged_calls,
    pin_cumsum_worked_example, pin_dt_zero, pin_split_resume, pin_step_equals_forward,
    pin_step_inputs_roundtrip, pin_linearity, pin_head_permutation, pin_groups,
    pin_frontend_softplus, pin_zoh_factor_matrix_exponential, pin_zoh_forward_solves_the_ode,
    pin_input_step_only_scales_the_input,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_zero_length_sequence():
    """L = 0 is a no-op that returns h0 as the final state."""
    fi = _small(seed=17, L=1)
    r = oracle.forward(fi.x[:, :0], fi.dt[:, :0], fi.A, fi.B[:, :0], fi.C[:, :0], fi.D, fi.h0)
    assert r["y"].shape[1] == 0
    assert np.array_equal(r["final"], fi.h0)


# ---------------------------------------------------------------------------
# planted mistakes: each must break at least one pin
# ---------------------------------------------------------------------------

MUTANTS = {
    "decay_sign": ("double a = exp(dt * A);", "double a = exp(-dt * A);"),
    "input_without_dt": ("double u = dtu * x[p];", "double u = x[p];"),
    "B_for_C_in_update": ("row[n] = a * row[n] + u * B[n];", "row[n] = a * row[n] + u * C[n];"),
    "dropped_D": ("y[p] = acc + (has_D ? Dh * x[p] : 0.0);", "y[p] = acc;"),
    "output_before_decay": ("double a = exp(dt * A);", "double a = 1.0;"),
    "transposed_state_read": ("for (int64_t n = 0; n < N; ++n) acc += C[n] * row[n];",
                              "for (int64_t n = 0; n < N; ++n) acc += C[n] * S[n * P + p];"),
    "wrong_group": ("g = h / hpg;", "g = h % G;"),
    "cumsum_natural_units": ("cs_log2[o] = run * LOG2E_D;", "cs_log2[o] = run;"),
    "cumsum_exclusive": ("run += d * A[h];\n                    int64_t o", "int64_t o"),
    "passing_first_decay": ("* Q + (Q - 1)]);", "* Q + 0]);"),
    "passing_start_after_update": (
        "if (chunk_start) memcpy(chunk_start + o, S, sizeof(double) * PN);\n                for (int64_t e = 0; e < PN; ++e) S[e] = decay * S[e] + tmp[e];",
        "for (int64_t e = 0; e < PN; ++e) S[e] = decay * S[e] + tmp[e];\n                if (chunk_start) memcpy(chunk_start + o, S, sizeof(double) * PN);",
    ),
    "chunk_start_off_by_one": ("if (chunk_start && t % chunk == 0)", "if (chunk_start && t % chunk == 1)"),
    "frontend_bias_dropped": ("if (bias) d = d + bias[h];", ""),
    "softplus_branch": ("d = d > 0.0 ? d + log1p(exp(-d)) : log1p(exp(d));",
                        "d = d > 0.0 ? log1p(exp(-d)) : log1p(exp(d));"),
    "zoh_without_division": ("in = expm1(d * A[h]) / A[h];", "in = expm1(d * A[h]);"),
    "decay_from_input_step": ("double a = exp(dt * A);", "double a = exp(dtu * A);"),
    "cumsum_ignores_input_step": ("if (dt_t) dt_t[o] = t < L && dt_in ? dt_in[(bb * L + t) * H + h] : d;",
                                  "if (dt_t) dt_t[o] = d;"),
}


def _build_mutant(src_text: str, tmpdir: str, name: str) -> str:
    src = os.path.join(tmpdir, f"{name}.c")
    lib = os.path.join(tmpdir, f"lib_{name}.so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-o", lib, src, "-lm"],
                   check=True)
    return lib


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed to build mutants")
def test_mutants_are_caught(monkeypatch):
    with open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")) as f:
        original = f.read()
    survivors = []
    with tempfile.TemporaryDirectory() as tmp:
        for name, (old, new) in MUTANTS.items():
            assert original.count(old) >= 1, f"mutation anchor for {name} not found in the oracle source"
            lib = _build_mutant(original.replace(old, new), tmp, name)
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
