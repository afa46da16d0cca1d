"""Python binding of libssd, the gfx950 Mamba-2 SSD chunked forward and decode step.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libssd.so``; PyTorch supplies device memory and the current
stream.  There is no CPU or PyTorch fallback -- if the library is not built,
``load()`` raises.

Calls (names follow the C ABI in ``include/ssd.h``):

    forward(x, dt, A, B, C, D=None, h0=None, chunk=0)       -> (y, final_state)
    step(state, x, dt, A, B, C, D=None)                    -> y   (state updated in place)
    chunk_cumsum(dt, A, chunk)                             -> (dt_t, dA_cs_log2)
    chunk_state(x, B, dt_t, dA_cs_log2, chunk)             -> states (chunk-local)
    state_passing(states, dA_cs_log2, h0=None, chunk=...)  -> (states -> chunk-start, final_state)
    chunk_scan(x, B, C, dt_t, dA_cs_log2, chunk_start, D=None, chunk=...) -> y

Layouts: x, y (b, L, H, P); dt (b, L, H); A, D (H); B, C (b, L, G, N);
h0, final and the decode state (b, H, P, N) float32; per-chunk (b, H, nC, Q)
and (b, nC, H, P, N) float32.  x, dt, B, C share one dtype: bfloat16 or float32.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "SsdError", "load", "library_path", "forward", "forward_noalloc", "forward_workspace_bytes", "step", "step_multi",
    "chunk_cumsum",
    "chunk_state", "state_passing", "chunk_scan", "query_config", "abi_version", "Dims", "DtFrontend",
    "Frontend",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssd.so")
_lib = None

SSD_OK, SSD_ERR_NULL, SSD_ERR_SHAPE, SSD_ERR_DTYPE, SSD_ERR_UNSUPPORTED, SSD_ERR_WORKSPACE, SSD_ERR_ALIAS, \
    SSD_ERR_HIP = range(8)
SSD_F32, SSD_BF16 = 0, 1


class SsdError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: status {status} ({detail})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
        ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
        ("chunk", ctypes.c_int64), ("io", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class DtFrontend(ctypes.Structure):
    _fields_ = [
        ("dt_bias", ctypes.c_void_p), ("softplus", ctypes.c_int32), ("zoh", ctypes.c_int32),
        ("clamp", ctypes.c_int32), ("reserved", ctypes.c_int32), ("dt_min", ctypes.c_float),
        ("dt_max", ctypes.c_float),
    ]


class Frontend:
    """The dt front-end of the *_ex calls: ``dt_bias`` (H) float32 GPU tensor or None, ``softplus``,
    ``zoh`` (zero-order-hold input step) and ``clamp`` = (dt_min, dt_max) or None."""

    def __init__(self, dt_bias: Optional[torch.Tensor] = None, softplus: bool = False, zoh: bool = False,
                 clamp: Optional[Tuple[float, float]] = None):
        self.dt_bias, self.softplus, self.zoh, self.clamp = dt_bias, softplus, zoh, clamp

    def _c(self, H: int) -> DtFrontend:
        _dev(self.dt_bias, "dt_bias", torch.float32, (H,))
        lo, hi = self.clamp if self.clamp is not None else (0.0, 0.0)
        return DtFrontend(_ptr(self.dt_bias), int(bool(self.softplus)), int(bool(self.zoh)),
                          int(self.clamp is not None), 0, float(lo), float(hi))


def _fe(frontend: Optional[Frontend], H: int):
    return None if frontend is None else ctypes.byref(frontend._c(H))


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libssd.so (built in-tree by ``build.py``); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libssd.so is not built ({_LIB_PATH}); run mamba_ssd_chunked_05_amd/build.py")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, dp, fp = ctypes.c_void_p, ctypes.POINTER(Dims), ctypes.POINTER(DtFrontend)
    sig = {
        "ssd_chunk_cumsum": [dp, vp, vp, vp, vp, vp],
        "ssd_chunk_state": [dp, vp, vp, vp, vp, vp, vp],
        "ssd_state_passing": [dp, vp, vp, vp, vp, vp],
        "ssd_chunk_scan": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "ssd_forward": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "ssd_step": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "ssd_step_multi": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "ssd_chunk_cumsum_ex": [dp, fp, vp, vp, vp, vp, vp],
        "ssd_forward_ex": [dp, fp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "ssd_forward_noalloc": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "ssd_bench_rmw_stream": [vp, ctypes.c_size_t, ctypes.c_float, ctypes.c_float, vp],
        "ssd_step_ex": [dp, fp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "ssd_step_multi_ex": [dp, fp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "ssd_query_config": [dp] + [ctypes.POINTER(ctypes.c_int)] * 4,
        "ssd_selective_scan": [dp, fp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp],
        "ssd_backward": [dp] + [vp] * 17 + [ctypes.c_size_t, vp],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ssd_forward_workspace_bytes.argtypes = [dp]
    lib.ssd_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_backward_workspace_bytes.argtypes = [dp]
    lib.ssd_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_selective_scan_workspace_bytes.argtypes = [dp]
    lib.ssd_selective_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.ssd_status_string.argtypes = [ctypes.c_int]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def abi_version() -> int:
    return int(load().ssd_abi_version())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

_IO = {torch.bfloat16: SSD_BF16, torch.float32: SSD_F32}


def _io_code(t: torch.Tensor) -> int:
    if t.dtype not in _IO:
        raise TypeError(f"x/dt/B/C must be bfloat16 or float32, got {t.dtype}")
    return _IO[t.dtype]


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() and t.data_ptr() % 16:
        raise ValueError(f"{name} must be 16-byte aligned")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None or t.numel() == 0 else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(status: int, func: str):
    if status != SSD_OK:
        lib = load()
        detail = lib.ssd_last_error().decode() or lib.ssd_status_string(status).decode()
        if status == SSD_ERR_HIP:
            raise SsdError(status, func, detail)
        raise ValueError(f"{func}: {lib.ssd_status_string(status).decode()}: {detail}")


def _dims(b, L, H, P, N, G, chunk, io) -> Dims:
    return Dims(int(b), int(L), int(H), int(P), int(N), int(G), int(chunk), int(io), 0)


def _fwd_dims(x, B, chunk):
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be (b, L, H, P) and B, C (b, L, G, N)")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return _dims(b, L, H, P, N, G, chunk, _io_code(x))


def _check_fwd_inputs(x, dt, A, B, C, D, h0):
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _dev(x, "x")
    _dev(dt, "dt", x.dtype, (b, L, H))
    _dev(A, "A", torch.float32, (H,))
    _dev(B, "B", x.dtype, (b, L, G, N))
    _dev(C, "C", x.dtype, (b, L, G, N))
    _dev(D, "D", torch.float32, (H,))
    _dev(h0, "h0", torch.float32, (b, H, P, N))


# ---------------------------------------------------------------------------
# the calls
# ---------------------------------------------------------------------------


def query_config(b, L, H, P, N, G=1, chunk=0, dtype=torch.bfloat16) -> dict:
    lib = load()
    d = _dims(b, L, H, P, N, G, chunk, _IO[dtype])
    out = [ctypes.c_int(0) for _ in range(4)]
    _check(lib.ssd_query_config(ctypes.byref(d), *[ctypes.byref(o) for o in out]), "ssd_query_config")
    return dict(chunk=out[0].value, tile_p=out[1].value, heads_per_wg=out[2].value,
                chunks_per_segment=out[3].value)


def forward_workspace_bytes(x: torch.Tensor, B: torch.Tensor, chunk: int = 0) -> int:
    lib = load()
    d = _fwd_dims(x, B, chunk)
    return int(lib.ssd_forward_workspace_bytes(ctypes.byref(d)))


def forward(x, dt, A, B, C, D=None, h0=None, *, chunk: int = 0, y=None, final_state=None,
            workspace=None, frontend: Optional[Frontend] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One-shot SSD forward on the current stream; returns (y, final_state).  ``frontend`` (optional)
    turns the raw dt into the step (bias, softplus, clamp, zero-order-hold input step)."""
    lib = load()
    d = _fwd_dims(x, B, chunk)
    _check_fwd_inputs(x, dt, A, B, C, D, h0)
    b, L, H, P = x.shape
    N = B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    if final_state is None:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    _dev(final_state, "final_state", torch.float32, (b, H, P, N))
    nbytes = int(lib.ssd_forward_workspace_bytes(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    st = lib.ssd_forward_ex(ctypes.byref(d), _fe(frontend, H), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                            _ptr(D), _ptr(h0), _ptr(y), _ptr(final_state), _ptr(workspace), workspace.numel(),
                            _stream(x))
    _check(st, "ssd_forward")
    return y, final_state


def forward_noalloc(x, dt, A, B, C, D=None, h0=None, *, chunk: int = 0, y=None,
                    final_state=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """ssd_forward_noalloc: the forward with the library's static device scratch instead of a workspace.
    Pass ``y`` and ``final_state`` to keep the call free of any allocation."""
    lib = load()
    d = _fwd_dims(x, B, chunk)
    _check_fwd_inputs(x, dt, A, B, C, D, h0)
    b, L, H, P = x.shape
    N = B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    if final_state is None:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    _dev(final_state, "final_state", torch.float32, (b, H, P, N))
    st = lib.ssd_forward_noalloc(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
                                 _ptr(y), _ptr(final_state), _stream(x))
    _check(st, "ssd_forward_noalloc")
    return y, final_state


def bench_rmw_stream(buf: torch.Tensor, a: float = 1.0, b: float = 0.0) -> None:
    """Measurement helper (ssd_bench.h): buf <- a * buf + b in place, float32, on the current stream."""
    lib = load()
    _dev(buf, "buf", torch.float32)
    _check(lib.ssd_bench_rmw_stream(_ptr(buf), buf.numel(), a, b, _stream(buf)), "ssd_bench_rmw_stream")


def step(state, x, dt, A, B, C, D=None, *, y=None, frontend: Optional[Frontend] = None) -> torch.Tensor:
    """One decode token per (b, h); ``state`` (b, H, P, N) float32 is updated in place."""
    lib = load()
    b, H, P, N = state.shape
    G = B.shape[1]
    _dev(state, "state", torch.float32)
    _dev(x, "x", None, (b, H, P))
    _dev(dt, "dt", x.dtype, (b, H))
    _dev(A, "A", torch.float32, (H,))
    _dev(B, "B", x.dtype, (b, G, N))
    _dev(C, "C", x.dtype, (b, G, N))
    _dev(D, "D", torch.float32, (H,))
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, (b, H, P))
    d = _dims(b, 1, H, P, N, G, 0, _io_code(x))
    st = lib.ssd_step_ex(ctypes.byref(d), _fe(frontend, H), _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                         _ptr(C), _ptr(D), _ptr(y), _stream(x))
    _check(st, "ssd_step")
    return y


def step_multi(state, x, dt, A, B, C, D=None, *, y=None, frontend: Optional[Frontend] = None) -> torch.Tensor:
    """K pre-staged decode steps: x (b, K, H, P), dt (b, K, H), B, C (b, K, G, N); ``state``
    (b, H, P, N) float32 is updated in place; returns y (b, K, H, P)."""
    lib = load()
    b, H, P, N = state.shape
    K = x.shape[1]
    G = B.shape[2]
    _dev(state, "state", torch.float32)
    _dev(x, "x", None, (b, K, H, P))
    _dev(dt, "dt", x.dtype, (b, K, H))
    _dev(A, "A", torch.float32, (H,))
    _dev(B, "B", x.dtype, (b, K, G, N))
    _dev(C, "C", x.dtype, (b, K, G, N))
    _dev(D, "D", torch.float32, (H,))
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, (b, K, H, P))
    d = _dims(b, K, H, P, N, G, 0, _io_code(x))
    st = lib.ssd_step_multi_ex(ctypes.byref(d), _fe(frontend, H), _ptr(state), _ptr(x), _ptr(dt), _ptr(A),
                               _ptr(B), _ptr(C), _ptr(D), _ptr(y), _stream(x))
    _check(st, "ssd_step_multi")
    return y


def backward_workspace_bytes(x: torch.Tensor, B: torch.Tensor, chunk: int = 0) -> int:
    d = _fwd_dims(x, B, chunk)
    return int(load().ssd_backward_workspace_bytes(ctypes.byref(d)))


def backward(x, dt, A, B, C, D=None, h0=None, dy=None, dfinal=None, *, chunk: int = 0, workspace=None) -> dict:
    """Gradients of ssd_forward (plain dt) for output gradient ``dy`` (layout of x) and final-state gradient
    ``dfinal`` (b, H, P, N) float32 or None.  Returns dict(dx, ddt, dA, dB, dC, dD, dh0): dx, ddt, dB, dC in
    the io dtype, dA, dD, dh0 float32 (dD None when D is None)."""
    lib = load()
    d = _fwd_dims(x, B, chunk)
    _check_fwd_inputs(x, dt, A, B, C, D, h0)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _dev(dy, "dy", x.dtype, x.shape)
    _dev(dfinal, "dfinal", torch.float32, (b, H, P, N))
    out = {
        "dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "dA": torch.empty((H,), dtype=torch.float32,
                                                                                 device=x.device),
        "dB": torch.empty_like(B), "dC": torch.empty_like(C),
        "dD": None if D is None else torch.empty((H,), dtype=torch.float32, device=x.device),
        "dh0": torch.empty((b, H, P, N), dtype=torch.float32, device=x.device),
    }
    nbytes = int(lib.ssd_backward_workspace_bytes(ctypes.byref(d)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    st = lib.ssd_backward(ctypes.byref(d), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), _ptr(dy),
                          _ptr(dfinal), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]),
                          _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dh0"]), _ptr(workspace), workspace.numel(),
                          _stream(x))
    _check(st, "ssd_backward")
    return out


def selective_scan_workspace_bytes(b, L, Dc, N, G=1, *, chunk: int = 0, dtype=torch.bfloat16) -> int:
    d = _dims(b, L, Dc, 1, N, G, chunk, _IO[dtype])
    return int(load().ssd_selective_scan_workspace_bytes(ctypes.byref(d)))


def selective_scan(x, delta, A, B, C, D=None, h0=None, *, chunk: int = 0, y=None, final_state=None,
                   workspace=None, frontend: Optional[Frontend] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Mamba-1 selective scan on the current stream: x, delta (b, L, Dc); A (Dc, N) float32; B, C
    (b, L, G, N); D (Dc,) and h0 (b, Dc, N) float32 or None.  ``frontend`` turns the raw delta into
    the step (per-channel bias, softplus, clamp) and its ``zoh`` flag selects the zero-order-hold
    input; without it the input is delta * B.  ``chunk`` is the segment length (0: the library's
    choice).  Returns (y, final_state)."""
    lib = load()
    if x.dim() != 3 or B.dim() != 4:
        raise ValueError("x must be (b, L, Dc) and B, C (b, L, G, N)")
    b, L, Dc = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x)
    _dev(x, "x")
    _dev(delta, "delta", x.dtype, (b, L, Dc))
    _dev(A, "A", torch.float32, (Dc, N))
    _dev(B, "B", x.dtype, (b, L, G, N))
    _dev(C, "C", x.dtype, (b, L, G, N))
    _dev(D, "D", torch.float32, (Dc,))
    _dev(h0, "h0", torch.float32, (b, Dc, N))
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, (b, L, Dc))
    if final_state is None:
        final_state = torch.empty((b, Dc, N), dtype=torch.float32, device=x.device)
    _dev(final_state, "final_state", torch.float32, (b, Dc, N))
    d = _dims(b, L, Dc, 1, N, G, chunk, io)
    nbytes = int(lib.ssd_selective_scan_workspace_bytes(ctypes.byref(d)))
    if workspace is None and nbytes > 0:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _dev(workspace, "workspace", torch.uint8)
    st = lib.ssd_selective_scan(ctypes.byref(d), _fe(frontend, Dc), _ptr(x), _ptr(delta), _ptr(A), _ptr(B),
                                _ptr(C), _ptr(D), _ptr(h0), _ptr(y), _ptr(final_state), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), _stream(x))
    _check(st, "ssd_selective_scan")
    return y, final_state


def chunk_cumsum(dt, A, chunk: int, *, frontend: Optional[Frontend] = None):
    lib = load()
    b, L, H = dt.shape
    _dev(dt, "dt")
    _dev(A, "A", torch.float32, (H,))
    nC = -(-L // chunk)
    dt_t = torch.empty((b, H, nC, chunk), dtype=torch.float32, device=dt.device)
    cs = torch.empty_like(dt_t)
    d = _dims(b, L, H, 16, 16, 1, chunk, _io_code(dt))
    _check(lib.ssd_chunk_cumsum_ex(ctypes.byref(d), _fe(frontend, H), _ptr(dt), _ptr(A), _ptr(dt_t), _ptr(cs),
                                   _stream(dt)), "ssd_chunk_cumsum")
    return dt_t, cs


def chunk_state(x, B, dt_t, cs, chunk: int):
    lib = load()
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nC = -(-L // chunk)
    _dev(x, "x")
    _dev(B, "B", x.dtype, (b, L, G, N))
    _dev(dt_t, "dt_t", torch.float32, (b, H, nC, chunk))
    _dev(cs, "dA_cs_log2", torch.float32, (b, H, nC, chunk))
    states = torch.empty((b, nC, H, P, N), dtype=torch.float32, device=x.device)
    d = _dims(b, L, H, P, N, G, chunk, _io_code(x))
    _check(lib.ssd_chunk_state(ctypes.byref(d), _ptr(x), _ptr(B), _ptr(dt_t), _ptr(cs), _ptr(states),
                               _stream(x)), "ssd_chunk_state")
    return states


def state_passing(states, cs, h0=None, *, seqlen: int, chunk: int, io=torch.bfloat16, final_state=None):
    """In place: chunk-local states -> chunk-start states.  Returns (states, final_state)."""
    lib = load()
    b, nC, H, P, N = states.shape
    _dev(states, "states", torch.float32)
    _dev(cs, "dA_cs_log2", torch.float32, (b, H, nC, chunk))
    _dev(h0, "h0", torch.float32, (b, H, P, N))
    if -(-seqlen // chunk) != nC:
        raise ValueError("states has the wrong number of chunks for seqlen/chunk")
    if final_state is None:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=states.device)
    _dev(final_state, "final_state", torch.float32, (b, H, P, N))
    d = _dims(b, seqlen, H, P, N, 1, chunk, _IO[io])
    _check(lib.ssd_state_passing(ctypes.byref(d), _ptr(states), _ptr(cs), _ptr(h0), _ptr(final_state),
                                 _stream(states)), "ssd_state_passing")
    return states, final_state


def chunk_scan(x, B, C, dt_t, cs, chunk_start, D=None, *, chunk: int, y=None):
    lib = load()
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nC = -(-L // chunk)
    _dev(x, "x")
    _dev(B, "B", x.dtype, (b, L, G, N))
    _dev(C, "C", x.dtype, (b, L, G, N))
    _dev(dt_t, "dt_t", torch.float32, (b, H, nC, chunk))
    _dev(cs, "dA_cs_log2", torch.float32, (b, H, nC, chunk))
    _dev(chunk_start, "chunk_start_states", torch.float32, (b, nC, H, P, N))
    _dev(D, "D", torch.float32, (H,))
    if y is None:
        y = torch.empty_like(x)
    _dev(y, "y", x.dtype, x.shape)
    d = _dims(b, L, H, P, N, G, chunk, _io_code(x))
    _check(lib.ssd_chunk_scan(ctypes.byref(d), _ptr(x), _ptr(B), _ptr(C), _ptr(dt_t), _ptr(cs),
                              _ptr(chunk_start), _ptr(D), _ptr(y), _stream(x)), "ssd_chunk_scan")
    return y
