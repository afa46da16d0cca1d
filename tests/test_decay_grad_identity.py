"""The chunk-local form of the backward's decay gradient (CPU, fp64, numpy only).

The decay gradient at token k is R_k = sum_{t>=k} dlambda_t with
dlambda_t = C_t . (S_t^T dy_t) - dt_t x_t^T G_t B_t (+ <dfinal, S_{L-1}> at the last
token), S the forward state and G the adjoint.  The GPU backward forms it chunk by chunk
as T1 + T2_k + T3_k + T4_k from the chunk-start state S0 and the adjoint Gam entering the
chunk from the next one.  Here both forms are computed from their definitions and must
agree for ragged chunks, sequences shorter than one chunk, with and without h0 and dfinal.
A planted mistake in the chunked form (a dropped term, an off-by-one in the box sum, a
missing decay of Gam) must break the agreement.  (M's diagonal would enter both its row
and column sums, so including it cannot be seen: the box takes j < t strictly, as the GPU
kernel does.)
"""

from __future__ import annotations

import numpy as np
import pytest


def _direct(x, dt, A, B, C, dy, h0, dfinal):
    L = x.shape[0]
    a = np.exp(dt * A)
    S = h0.copy()
    w = np.zeros((L, B.shape[1]))
    for t in range(L):
        S = a[t] * S + dt[t] * np.outer(x[t], B[t])
        w[t] = S.T @ dy[t]
    G = dfinal.copy()
    v = np.zeros_like(w)
    for t in range(L - 1, -1, -1):
        if t < L - 1:
            G = a[t + 1] * G
        G = G + np.outer(dy[t], C[t])
        v[t] = G.T @ x[t]
    dlam = np.sum(C * w, axis=1) - dt * np.sum(v * B, axis=1)
    dlam[-1] += np.sum(dfinal * S)
    return np.cumsum(dlam[::-1])[::-1]


def _chunked(x, dt, A, B, C, dy, h0, dfinal, Q, mistake=None):
    L = x.shape[0]
    nC = (L + Q - 1) // Q
    a = np.exp(dt * A)
    S = h0.copy()
    S0 = []
    for c in range(nC):
        S0.append(S.copy())
        for t in range(c * Q, min(L, (c + 1) * Q)):
            S = a[t] * S + dt[t] * np.outer(x[t], B[t])
    Gam = [None] * nC
    G = dfinal.copy()
    for c in range(nC - 1, -1, -1):
        c0, c1 = c * Q, min(L, (c + 1) * Q) - 1
        Gam[c] = G.copy()  # a_{c1+1} G_{c1+1}; dfinal for the last chunk
        for t in range(c1, c0 - 1, -1):
            G = G + np.outer(dy[t], C[t])
            if t > c0 or mistake != "gam_decay":
                G = a[t] * G
    R = np.zeros(L)
    for c in range(nC):
        c0, c1 = c * Q, min(L, (c + 1) * Q) - 1
        sl = slice(c0, c1 + 1)
        l = np.cumsum(dt[sl] * A)
        T1 = np.exp(l[-1]) * np.sum(Gam[c] * S0[c])
        s2 = np.exp(l) * np.sum(dy[sl] * (C[sl] @ S0[c].T), axis=1)
        T2 = np.cumsum(s2[::-1])[::-1]
        s3 = dt[sl] * np.exp(l[-1] - l) * np.sum(x[sl] * (B[sl] @ Gam[c].T), axis=1)
        T3 = np.concatenate([[0.0], np.cumsum(s3)[:-1]])
        M = (dy[sl] @ x[sl].T) * (C[sl] @ B[sl].T) * np.exp(l[:, None] - l[None, :]) * dt[sl][None, :]
        M = np.tril(M, -1)
        T4 = np.concatenate([[0.0], np.cumsum(M.sum(axis=0) - M.sum(axis=1))[:-1]])
        if mistake == "box_inclusive":
            T4 = np.cumsum(M.sum(axis=0) - M.sum(axis=1))
        if mistake == "no_T3":
            T3 = 0.0
        R[sl] = T1 + T2 + T3 + T4
    return R


def _inputs(L, P, N, seed, with_state):
    rng = np.random.default_rng(seed)
    x, dy = rng.standard_normal((L, P)), rng.standard_normal((L, P))
    B, C = rng.standard_normal((L, N)), rng.standard_normal((L, N))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(0.5), L))
    A = -rng.uniform(1.0, 8.0)
    h0 = rng.standard_normal((P, N)) if with_state else np.zeros((P, N))
    dfinal = rng.standard_normal((P, N)) if with_state else np.zeros((P, N))
    return x, dt, A, B, C, dy, h0, dfinal


@pytest.mark.parametrize("L,P,N,Q,with_state", [(37, 4, 3, 8, True), (64, 5, 6, 16, True), (100, 3, 4, 32, False),
                                                (129, 8, 8, 64, True), (7, 2, 2, 16, True)])
def test_chunked_decay_gradient_matches_suffix_sums(L, P, N, Q, with_state):
    args = _inputs(L, P, N, 40 + L, with_state)
    R = _direct(*args)
    Rc = _chunked(*args, Q)
    assert np.max(np.abs(Rc - R)) <= 1e-12 * np.max(np.abs(R))


@pytest.mark.parametrize("mistake", ["gam_decay", "box_inclusive", "no_T3"])
def test_planted_mistakes_break_it(mistake):
    args = _inputs(70, 4, 5, 9, True)
    R = _direct(*args)
    Rc = _chunked(*args, 16, mistake=mistake)
    assert np.max(np.abs(Rc - R)) > 1e-6 * np.max(np.abs(R))
