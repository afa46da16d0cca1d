"""NumPy fp64 forms of the SSD forward, for tiny inputs only.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).  These pin the C recurrence
by brute force; they are three different ways of writing the same result:

* ``materialized``: every state S_t written out independently from its unrolled
  sum -- the (B, L, D, N) state tensor that the hardware-aware method avoids
  building ("3.3 Hardware-Aware algorithms and GPU memory hierarchy
  optimisation", section 2.1, state materialisation).
* ``quadratic``: the output as one lower-triangular (semiseparable) matrix
  applied to x along the sequence, plus the initial-state term.
* ``chunked``: the chunked decomposition in fp64 at any chunk size Q -- in-chunk
  cumulative sum of dt*A, chunk-local states, chunk-order state passing, and the
  chunk output from the chunk-start state (devotd.net page on the cuTile
  Mamba-2 forward kernels, sections 1 and 2).  Q = 1 is the recurrence and Q = L
  is the quadratic form.

Segment sums in ``materialized`` and ``quadratic`` are accumulated directly
(sum over k = s+1..t), never as a difference of two prefix sums, so they do not
share the cancellation pattern of the chunked method.
"""

from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)


def _segment_sums(dt: np.ndarray) -> np.ndarray:
    """seg[t, s] = sum_{k=s+1..t} dt_k for s <= t (0 on the diagonal); NaN above it."""
    L = dt.shape[0]
    seg = np.full((L, L), np.nan)
    for t in range(L):
        seg[t, t] = 0.0
        run = 0.0
        for s in range(t - 1, -1, -1):
            run += dt[s + 1]
            seg[t, s] = run
    return seg


def _prefix_sums(dt: np.ndarray) -> np.ndarray:
    """pre[t] = sum_{k=0..t} dt_k, accumulated directly."""
    out = np.empty(dt.shape[0])
    run = 0.0
    for t in range(dt.shape[0]):
        run += dt[t]
        out[t] = run
    return out


def _group(h: int, H: int, G: int) -> int:
    return h // (H // G)


def materialized(x, dt, A, B, C, D=None, h0=None):
    """Returns (y, final, states) with states (b, L, H, P, N) all written out."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros((b, L, H, P))
    states = np.zeros((b, L, H, P, N))
    for bb in range(b):
        for h in range(H):
            g = _group(h, H, G)
            d = dt[bb, :, h]
            seg = _segment_sums(d)
            pre = _prefix_sums(d)
            for t in range(L):
                S = np.zeros((P, N))
                if h0 is not None:
                    S += math.exp(A[h] * pre[t]) * h0[bb, h]
                for s in range(t + 1):
                    w = math.exp(A[h] * seg[t, s]) * d[s]
                    S += w * np.outer(x[bb, s, h], B[bb, s, g])
                states[bb, t, h] = S
                y[bb, t, h] = S @ C[bb, t, g]
                if D is not None:
                    y[bb, t, h] += D[h] * x[bb, t, h]
    if L > 0:
        final = states[:, L - 1].copy()
    else:
        final = np.zeros((b, H, P, N)) if h0 is None else np.array(h0, dtype=np.float64)
    return y, final, states


def quadratic(x, dt, A, B, C, D=None, h0=None):
    """y = M x + (initial-state term) + D x with M[t,s] = (C_t.B_s) exp(A seg[t,s]) dt_s, s <= t."""
    b, L, H, P = x.shape
    G = B.shape[2]
    y = np.zeros((b, L, H, P))
    for bb in range(b):
        for h in range(H):
            g = _group(h, H, G)
            d = dt[bb, :, h]
            seg = _segment_sums(d)
            mask = np.tril(np.ones((L, L), dtype=bool))
            decay = np.where(mask, np.exp(A[h] * np.where(mask, seg, 0.0)), 0.0)
            M = (C[bb, :, g] @ B[bb, :, g].T) * decay * d[None, :]
            yy = M @ x[bb, :, h]
            if h0 is not None:
                pre = _prefix_sums(d)
                yy += np.exp(A[h] * pre)[:, None] * (C[bb, :, g] @ h0[bb, h].T)
            if D is not None:
                yy += D[h] * x[bb, :, h]
            y[bb, :, h] = yy
    return y


def chunked(x, dt, A, B, C, D=None, h0=None, *, Q: int):
    """fp64 chunked form.  Returns dict(y, final, cs_log2, chunk_local, chunk_start)."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nC = -(-L // Q) if L > 0 else 0
    Lp = nC * Q
    # zero padding of the ragged tail: dt = 0 adds nothing and decays nothing
    xp = np.zeros((b, Lp, H, P)); xp[:, :L] = x
    dtp = np.zeros((b, Lp, H)); dtp[:, :L] = dt
    Bp = np.zeros((b, Lp, G, N)); Bp[:, :L] = B
    Cp = np.zeros((b, Lp, G, N)); Cp[:, :L] = C
    cs = np.zeros((b, H, nC, Q))
    local = np.zeros((b, nC, H, P, N))
    start = np.zeros((b, nC, H, P, N))
    final = np.zeros((b, H, P, N))
    yp = np.zeros((b, Lp, H, P))
    for bb in range(b):
        for h in range(H):
            g = _group(h, H, G)
            S = np.zeros((P, N)) if h0 is None else np.array(h0[bb, h], dtype=np.float64)
            for c in range(nC):
                sl = slice(c * Q, (c + 1) * Q)
                d = dtp[bb, sl, h]
                csc = np.cumsum(d * A[h])  # in-chunk cumulative sum (natural log)
                cs[bb, h, c] = csc * LOG2E
                X, Bc, Cc = xp[bb, sl, h], Bp[bb, sl, g], Cp[bb, sl, g]
                # chunk-local state: decay from token j to the chunk end
                w_end = np.exp(csc[-1] - csc) * d
                local[bb, c, h] = (X * w_end[:, None]).T @ Bc
                # chunk output: in-chunk causal part + chunk-start state part
                diff = csc[:, None] - csc[None, :]
                mask = np.tril(np.ones((Q, Q), dtype=bool))
                Lmat = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
                Mc = (Cc @ Bc.T) * Lmat * d[None, :]
                yc = Mc @ X + np.exp(csc)[:, None] * (Cc @ S.T)
                if D is not None:
                    yc += D[h] * X
                yp[bb, sl, h] = yc
                start[bb, c, h] = S
                S = math.exp(csc[-1]) * S + local[bb, c, h]
            final[bb, h] = S
    return {"y": yp[:, :L], "final": final, "cs_log2": cs, "chunk_local": local, "chunk_start": start}
