"""fp64 CPU oracle for the Mamba-2 SSD forward scan, its decode step and the Mamba-1 selective scan.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``mamba_ssd_chunked_05_amd``) and the library never
imports it.

Two independent implementations live here:

* ``libssd_oracle.so`` (``ssd_oracle.c``): the token-by-token fp64 recurrence,
  plus the plain definition of each staged call of the chunked forward.  This
  is what GPU results are compared against.
* ``ssd_ref`` (NumPy, tiny inputs only): the fully materialised state tensor,
  the quadratic (semiseparable) form and the fp64 chunked form.  They pin the
  C oracle by brute force.

Pins for every function (closed forms, brute force, invariants) are in
``tests/test_oracle_pins.py``; none is "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None

_I64 = ctypes.c_int64
_DP = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, no contraction, OpenMP over slices)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.ssd_oracle_forward.argtypes = [_I64] * 6 + [_DP] * 10 + [_I64, _DP, _DP, ctypes.c_int]
        lib.ssd_oracle_step.argtypes = [_I64] * 5 + [_DP] * 9 + [ctypes.c_int]
        lib.ssd_oracle_chunk_cumsum.argtypes = [_I64] * 4 + [_DP] * 5
        lib.ssd_oracle_dt_frontend.argtypes = ([_I64] * 2 + [_DP] * 3 + [ctypes.c_int] * 3
                                               + [ctypes.c_double] * 2 + [_DP] * 2)
        lib.ssd_oracle_state_passing.argtypes = [_I64] * 6 + [_DP] * 5
        lib.ssd_oracle_chunk_scan.argtypes = [_I64] * 7 + [_DP] * 8 + [ctypes.c_int]
        lib.ssd_oracle_selective_scan.argtypes = [_I64] * 5 + [_DP] * 9 + [ctypes.c_int] * 2
        lib.ssd_oracle_backward.argtypes = [_I64] * 6 + [_DP] * 16 + [ctypes.c_int]
        for f in ("ssd_oracle_forward", "ssd_oracle_step", "ssd_oracle_chunk_cumsum",
                  "ssd_oracle_state_passing", "ssd_oracle_chunk_scan", "ssd_oracle_dt_frontend",
                  "ssd_oracle_selective_scan", "ssd_oracle_backward"):
            getattr(lib, f).restype = ctypes.c_int
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _in(a: Optional[np.ndarray]):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=np.float64)
    return arr, arr.ctypes.data_as(_DP)


def _out(shape):
    arr = np.zeros(shape, dtype=np.float64)
    return arr, arr.ctypes.data_as(_DP)


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError(f"{name}: oracle rejected the arguments (rc={rc})")


def dt_frontend(raw, A, bias=None, *, softplus: bool = False, zoh: bool = False, clamp=None):
    """(dt_decay, dt_input) from a raw step (..., H): bias, softplus, clamp (lo, hi), and the
    zero-order-hold input factor (exp(dt A) - 1) / A when ``zoh``."""
    raw = np.asarray(raw, dtype=np.float64)
    H = raw.shape[-1]
    n = raw.size // H if H else 0
    ra, pr = _in(raw)
    Aa, pA = _in(A)
    ba, pb = _in(bias)
    dec, pd = _out(raw.shape)
    inp, pi = _out(raw.shape)
    lo, hi = (clamp if clamp is not None else (0.0, 0.0))
    rc = _load().ssd_oracle_dt_frontend(n, H, pr, pA, pb, int(softplus), int(zoh), int(clamp is not None),
                                        float(lo), float(hi), pd, pi)
    _check(rc, "dt_frontend")
    return dec, inp


def forward(x, dt, A, B, C, D=None, h0=None, *, dt_in=None, chunk: int = 0, chunk_states: bool = False,
            threads: int = 0):
    """Token recurrence.  Returns dict(y, final[, chunk_start, chunk_local]).  ``dt`` is the decay
    step; ``dt_in`` (default: dt) the step of the input term."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    keep = []
    ptrs = []
    for a in (x, dt, dt_in, A, B, C, D, h0):
        arr, p = _in(a)
        keep.append(arr)
        ptrs.append(p)
    y, py = _out((b, L, H, P))
    fin, pf = _out((b, H, P, N))
    res = {"y": y, "final": fin}
    pcs = pcl = None
    if chunk_states:
        if chunk <= 0:
            raise ValueError("chunk_states needs chunk > 0")
        nC = -(-L // chunk)
        res["chunk_start"], pcs = _out((b, nC, H, P, N))
        res["chunk_local"], pcl = _out((b, nC, H, P, N))
    rc = _load().ssd_oracle_forward(b, L, H, P, N, G, *ptrs, py, pf, chunk, pcs, pcl, threads)
    _check(rc, "forward")
    return res


def step(state, x, dt, A, B, C, D=None, *, dt_in=None, threads: int = 0):
    """One decode step.  ``state`` (b,H,P,N) float64 is updated in place; returns y (b,H,P).
    ``dt`` is the decay step, ``dt_in`` (default: dt) the step of the input term."""
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise TypeError("state must be a C-contiguous float64 array (updated in place)")
    b, H, P, N = state.shape
    G = B.shape[1]
    keep = []
    ptrs = []
    for a in (x, dt, dt_in, A, B, C, D):
        arr, p = _in(a)
        keep.append(arr)
        ptrs.append(p)
    y, py = _out((b, H, P))
    rc = _load().ssd_oracle_step(b, H, P, N, G, state.ctypes.data_as(_DP), *ptrs, py, threads)
    _check(rc, "step")
    return y


def chunk_cumsum(dt, A, chunk: int, *, dt_in=None):
    """(dt_t, cs_log2), both (b,H,nC,Q); dt_t is the input step (``dt_in`` when given)."""
    b, L, H = dt.shape
    nC = -(-L // chunk)
    dta, pdt = _in(dt)
    dia, pdi = _in(dt_in)
    Aa, pA = _in(A)
    dtt, pdtt = _out((b, H, nC, chunk))
    cs, pcs = _out((b, H, nC, chunk))
    _check(_load().ssd_oracle_chunk_cumsum(b, L, H, chunk, pdt, pdi, pA, pdtt, pcs), "chunk_cumsum")
    return dtt, cs


def state_passing(local, cs_log2, h0=None):
    """(chunk_start, final) from chunk-local states (b,nC,H,P,N) and the log2 cumsum."""
    b, nC, H, P, N = local.shape
    Q = cs_log2.shape[-1]
    la, pl = _in(local)
    ca, pc = _in(cs_log2)
    ha, ph = _in(h0)
    start, ps = _out((b, nC, H, P, N))
    fin, pf = _out((b, H, P, N))
    _check(_load().ssd_oracle_state_passing(b, nC, H, P, N, Q, pl, pc, ph, ps, pf), "state_passing")
    return start, fin


def chunk_scan(x, dt, A, B, C, chunk_start, D=None, *, chunk: int, threads: int = 0):
    """y (b,L,H,P): the recurrence over each chunk from its chunk-start state."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    keep = []
    ptrs = []
    for a in (x, dt, A, B, C, D, chunk_start):
        arr, p = _in(a)
        keep.append(arr)
        ptrs.append(p)
    y, py = _out((b, L, H, P))
    rc = _load().ssd_oracle_chunk_scan(b, L, H, P, N, G, chunk, *ptrs, py, threads)
    _check(rc, "chunk_scan")
    return y


def selective_scan(x, delta, A, B, C, D=None, h0=None, *, zoh: bool = True, threads: int = 0):
    """Mamba-1 selective scan by the token recurrence.  x, delta (b,L,Dc); A (Dc,N); B, C (b,L,G,N);
    D (Dc,) or None; h0 (b,Dc,N) or None.  ``delta`` is the step after any front-end; ``zoh`` picks
    the zero-order-hold input matrix (else delta * B).  Returns dict(y, final)."""
    b, L, Dc = x.shape
    G, N = B.shape[2], B.shape[3]
    keep = []
    ptrs = []
    for a in (x, delta, A, B, C, D, h0):
        arr, p = _in(a)
        keep.append(arr)
        ptrs.append(p)
    y, py = _out((b, L, Dc))
    fin, pf = _out((b, Dc, N))
    rc = _load().ssd_oracle_selective_scan(b, L, Dc, N, G, *ptrs, py, pf, int(zoh), threads)
    _check(rc, "selective_scan")
    return {"y": y, "final": fin}


def backward(x, dt, A, B, C, D, h0, dy, dfinal=None, *, threads: int = 0):
    """Gradients of the SSD forward (plain input step dt) for output gradient dy (b,L,H,P) and final-state
    gradient dfinal (b,H,P,N) or None.  Returns dict(dx, ddt, dA, dB, dC, dD, dh0); dD is None when D is."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    keep = []
    ptrs = []
    for a in (x, dt, A, B, C, D, h0, dy, dfinal):
        arr, p = _in(a)
        keep.append(arr)
        ptrs.append(p)
    dx, pdx = _out((b, L, H, P))
    ddt, pddt = _out((b, L, H))
    dA, pdA = _out((H,))
    dB, pdB = _out((b, L, G, N))
    dC, pdC = _out((b, L, G, N))
    dD, pdD = _out((H,)) if D is not None else (None, None)
    dh0, pdh0 = _out((b, H, P, N))
    rc = _load().ssd_oracle_backward(b, L, H, P, N, G, *ptrs, pdx, pddt, pdA, pdB, pdC, pdD, pdh0, threads)
    _check(rc, "backward")
    return {"dx": dx, "ddt": ddt, "dA": dA, "dB": dB, "dC": dC, "dD": dD, "dh0": dh0}
