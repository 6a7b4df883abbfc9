"""ctypes binding of librosa (include/rosa.h).

Argument marshalling only: every function here passes device pointers,
sizes and the current HIP stream of torch to the C-ABI function of the same
name; all work runs in librosa's HIP kernels.  torch supplies device memory
and streams.  There is no CPU fallback: if librosa.so is missing or cannot
be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librosa.so")

ROSA_OK, ROSA_ERR_ARG, ROSA_ERR_CAPACITY, ROSA_ERR_SYMBOL, ROSA_ERR_HIP, \
    ROSA_ERR_STATE, ROSA_ERR_NOMEM = range(7)
# size of the fixed device array behind rosa_match_noalloc
ROSA_NOALLOC_MAX_WORKSPACE_BYTES = 96 << 20
ROSA_IN_SYMBOLS, ROSA_IN_BF16 = 0, 1
ROSA_QK_RLE = 1


class RosaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {rosa_error_string(status)} (status {status})")


class rosa_input(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("M", ctypes.c_int32),
                ("K", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("data", ctypes.c_void_p), ("S", ctypes.c_int64),
                ("T", ctypes.c_int64), ("B", ctypes.c_int64),
                ("D", ctypes.c_int64), ("ld", ctypes.c_int64)]


class rosa_out(ctypes.Structure):
    _fields_ = [("end", ctypes.c_void_p), ("sym", ctypes.c_void_p),
                ("len", ctypes.c_void_p), ("symbols", ctypes.c_void_p)]


class rosa_qk_out(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("tau", "end", "len", "run_of", "run_start", "ridx", "cf_tau",
                 "cf_ridx")]


_lib = None
_SYMBOLS = ["rosa_discretize", "rosa_match_workspace_bytes", "rosa_match", "rosa_match_timed",
            "rosa_match_status", "rosa_match_noalloc", "rosa_match_qk_workspace_bytes",
            "rosa_match_qk", "rosa_scatter_grad_workspace_bytes",
            "rosa_scatter_grad",
            "rosa_gather", "rosa_state_bytes", "rosa_build", "rosa_step",
            "rosa_qk_state_bytes", "rosa_build_qk", "rosa_step_qk",
            "rosa_state_length", "rosa_state_status", "rosa_free",
            "rosa_error_string"]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librosa.so and declare the C-ABI signatures (no GPU needed)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"librosa.so not built at {path}; run "
                           "__graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                       ctypes.c_size_t)
    sig = {
        "rosa_discretize": ([P, P, I64, P], ctypes.c_int),
        "rosa_match_workspace_bytes": ([I64, I64, I32], SZ),
        "rosa_match": ([P, P, P, SZ, P], ctypes.c_int),
        "rosa_match_timed": ([P, P, P, SZ, P, P, P], ctypes.c_int),
        "rosa_match_status": ([P, P], ctypes.c_int),
        "rosa_match_noalloc": ([P, P, P], ctypes.c_int),
        "rosa_match_qk_workspace_bytes": ([I64, I64, I32], SZ),
        "rosa_match_qk": ([P, P, I32, P, P, SZ, P], ctypes.c_int),
        "rosa_scatter_grad_workspace_bytes": ([I64, I64], SZ),
        "rosa_scatter_grad": ([P, I64, I64, I64, I64, I32, P, P, I64, P, SZ, P],
                              ctypes.c_int),
        "rosa_gather": ([P, I64, I64, I64, I64, I32, P, P, I64, P], ctypes.c_int),
        "rosa_state_bytes": ([I64, I32, I64], SZ),
        "rosa_build": ([P, I64, P, SZ, ctypes.POINTER(P), P, P], ctypes.c_int),
        "rosa_step": ([P, P, P, I64, I64, P, P, P, I64, P], ctypes.c_int),
        "rosa_qk_state_bytes": ([I64, I32, I64], SZ),
        "rosa_build_qk": ([P, P, I32, I64, P, SZ, ctypes.POINTER(P), P, P],
                          ctypes.c_int),
        "rosa_step_qk": ([P, P, P, P, P], ctypes.c_int),
        "rosa_state_length": ([P], I64),
        "rosa_state_status": ([P, P], ctypes.c_int),
        "rosa_free": ([P], None),
        "rosa_error_string": ([ctypes.c_int], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def rosa_error_string(status: int) -> str:
    return load_library().rosa_error_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != ROSA_OK:
        raise RosaError(status, what)


# torch's raw current-stream query (a fraction of a microsecond, against a
# few for torch.cuda.current_stream(), which builds a Stream object); the
# public call is the fallback where the private one is absent
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device: torch.device | None = None) -> ctypes.c_void_p:
    """The caller's stream, else the current stream of `device` (of the
    current device when None)."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is not None:
        idx = device.index if device is not None and device.index is not None \
            else torch.cuda.current_device()
        return ctypes.c_void_p(_raw_stream(idx))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _require_device(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("librosa takes device tensors only")


# -------------------------------------------------------------- inputs

def symbols_input(sym: torch.Tensor, K: int) -> rosa_input:
    """uint8 symbols [S, T] (rows may be padded: stride(0) >= T)."""
    _require_device(sym)
    if sym.dtype != torch.uint8 or sym.dim() != 2 or sym.stride(1) != 1:
        raise ValueError("symbols must be a uint8 [S, T] tensor, unit stride in T")
    inp = rosa_input()
    inp.kind, inp.K = ROSA_IN_SYMBOLS, int(K)
    inp.data = sym.data_ptr()
    inp.S, inp.T = sym.shape
    inp.ld = sym.stride(0) if sym.shape[0] > 1 else max(sym.shape[1], 1)
    inp._keep = sym
    return inp


def bf16_input(H: torch.Tensor, M: int) -> rosa_input:
    """bf16 (or int16 bit patterns) hidden states [B, T, D], unit stride in D,
    rows of stride ld = stride(1) elements and batch stride T*ld."""
    _require_device(H)
    if H.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or H.dim() != 3:
        raise ValueError("H must be a 16-bit [B, T, D] tensor")
    B, T, D = H.shape
    if H.stride(2) != 1 or (B > 1 and H.stride(0) != T * H.stride(1)):
        raise ValueError("H must be [B][T][ld] with unit channel stride")
    inp = rosa_input()
    inp.kind, inp.M = ROSA_IN_BF16, int(M)
    inp.data = H.data_ptr()
    inp.B, inp.T, inp.D = B, T, D
    inp.ld = H.stride(1) if T > 1 else D
    inp._keep = H
    return inp


def make_out(end, sym=None, len=None, symbols=None) -> rosa_out:
    _require_device(end, sym, len, symbols)
    o = rosa_out()
    o.end, o.sym, o.len, o.symbols = _ptr(end), _ptr(sym), _ptr(len), _ptr(symbols)
    return o


# ------------------------------------------------------ C-ABI functions

def rosa_discretize(inp: rosa_input, symbols: torch.Tensor, stream=None) -> None:
    """The symbols of a bf16 input alone: uint8 [S, T] rows (unit stride in
    T, row stride >= T) for S = B*D/M streams."""
    _require_device(symbols)
    if symbols.dtype != torch.uint8 or symbols.dim() != 2 or symbols.stride(1) != 1 \
            or tuple(symbols.shape) != (inp.B * (inp.D // max(inp.M, 1)), inp.T):
        raise ValueError("symbols must be a uint8 [B*D/M, T] tensor, unit stride in T")
    ld = symbols.stride(0) if symbols.shape[0] > 1 else max(inp.T, 1)
    _check(load_library().rosa_discretize(ctypes.byref(inp), symbols.data_ptr(), ld,
                                          _stream(stream)), "rosa_discretize")


def rosa_match_workspace_bytes(S: int, T: int, K: int) -> int:
    return int(load_library().rosa_match_workspace_bytes(S, T, K))


def rosa_match(inp: rosa_input, out: rosa_out, ws: torch.Tensor,
               stream=None) -> None:
    _require_device(ws)
    _check(load_library().rosa_match(ctypes.byref(inp), ctypes.byref(out),
                                     ws.data_ptr(), ws.numel() * ws.element_size(),
                                     _stream(stream)), "rosa_match")


def rosa_match_timed(inp: rosa_input, out: rosa_out, ws: torch.Tensor,
                     ev_begin: torch.cuda.Event, ev_end: torch.cuda.Event,
                     stream=None) -> None:
    """rosa_match that also records two torch (HIP) events around the
    retrieval kernel on the same stream."""
    _require_device(ws)
    for ev in (ev_begin, ev_end):
        if not ev.cuda_event:      # torch creates the HIP event on first record
            ev.record(stream if stream is not None else torch.cuda.current_stream())
    _check(load_library().rosa_match_timed(
        ctypes.byref(inp), ctypes.byref(out), ws.data_ptr(),
        ws.numel() * ws.element_size(), _stream(stream),
        ctypes.c_void_p(ev_begin.cuda_event), ctypes.c_void_p(ev_end.cuda_event)),
        "rosa_match_timed")


def rosa_match_noalloc(inp: rosa_input, out: rosa_out, stream=None) -> None:
    """rosa_match in the library's fixed device array: no workspace argument
    and no allocation (shapes whose workspace exceeds
    ROSA_NOALLOC_MAX_WORKSPACE_BYTES raise with ROSA_ERR_CAPACITY)."""
    _check(load_library().rosa_match_noalloc(ctypes.byref(inp), ctypes.byref(out),
                                             _stream(stream)),
           "rosa_match_noalloc")


def rosa_match_qk_workspace_bytes(S: int, T: int, K: int) -> int:
    return int(load_library().rosa_match_qk_workspace_bytes(S, T, K))


def make_qk_out(tau, **opt) -> rosa_qk_out:
    """tau: int32 [S, T]; optional end, len, run_of, run_start, ridx (int32
    [S, T]) and cf_tau, cf_ridx (int32 [S, T, M, 2])."""
    _require_device(tau, *opt.values())
    o = rosa_qk_out()
    o.tau = _ptr(tau)
    for name, t in opt.items():
        if name not in dict(rosa_qk_out._fields_):
            raise ValueError(f"unknown output {name}")
        setattr(o, name, _ptr(t))
    return o


def rosa_match_qk(q: rosa_input, k: rosa_input, flags: int, out: rosa_qk_out,
                  ws: torch.Tensor, stream=None) -> None:
    _require_device(ws)
    _check(load_library().rosa_match_qk(
        ctypes.byref(q), ctypes.byref(k), flags, ctypes.byref(out),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
        "rosa_match_qk")


def rosa_match_status(ws: torch.Tensor, stream=None) -> int:
    return int(load_library().rosa_match_status(ws.data_ptr(), _stream(stream)))


def _rows_3d(x: torch.Tensor, what: str, shape=None) -> None:
    """x must be [B, T, D] with unit channel stride and rows of one pitch
    (batch stride T * row stride), the layout the C-ABI reads and writes."""
    if x.dim() != 3 or (shape is not None and tuple(x.shape) != tuple(shape)):
        raise ValueError(f"{what} must be a [B, T, D] tensor"
                         + (f" of shape {tuple(shape)}" if shape is not None else ""))
    B, T, D = x.shape
    if x.stride(2) != 1 or (T > 1 and x.stride(1) < D) or \
            (B > 1 and x.stride(0) != T * x.stride(1)):
        raise ValueError(f"{what} must be [B][T][ld] with unit channel stride "
                         "and batch stride T * ld")


def _end_rows(end: torch.Tensor, S: int, T: int) -> None:
    if end.dtype != torch.int32 or tuple(end.shape) != (S, T) or \
            (T > 0 and not end.is_contiguous()):
        raise ValueError(f"end must be a contiguous int32 [{S}, {T}] tensor")


def rosa_gather(V: torch.Tensor, M: int, end: torch.Tensor, out: torch.Tensor,
                stream=None) -> None:
    """V, out: 16-bit [B, T, D] (unit channel stride); end: int32 [S, T]."""
    _require_device(V, end, out)
    if V.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or \
            out.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("V and out must be 16-bit tensors")
    _rows_3d(V, "V")
    _rows_3d(out, "out", V.shape)
    B, T, D = V.shape
    if M < 1 or D % M:
        raise ValueError("D must be a multiple of M")
    _end_rows(end, B * (D // M), T)
    _check(load_library().rosa_gather(V.data_ptr(), B, T, D,
                                      V.stride(1) if T > 1 else D, M,
                                      end.data_ptr(), out.data_ptr(),
                                      out.stride(1) if T > 1 else D,
                                      _stream(stream)), "rosa_gather")


def rosa_scatter_grad_workspace_bytes(S: int, T: int) -> int:
    return int(load_library().rosa_scatter_grad_workspace_bytes(S, T))


def rosa_scatter_grad(theta: torch.Tensor, M: int, end: torch.Tensor,
                      G: torch.Tensor, ws: torch.Tensor | None = None,
                      stream=None) -> None:
    """theta, G: float32 [B, T, D] (unit channel stride); end: int32 [S, T].
    Allocates the workspace with torch when none is given."""
    _require_device(theta, end, G, ws)
    if theta.dtype != torch.float32 or G.dtype != torch.float32:
        raise ValueError("theta and G must be float32")
    _rows_3d(theta, "theta")
    _rows_3d(G, "G", theta.shape)
    B, T, D = theta.shape
    if M < 1 or D % M:
        raise ValueError("D must be a multiple of M")
    _end_rows(end, B * (D // M), T)
    if ws is None:
        ws = torch.empty(rosa_scatter_grad_workspace_bytes(B * (D // M), T),
                         dtype=torch.uint8, device=theta.device)
    _check(load_library().rosa_scatter_grad(
        theta.data_ptr(), B, T, D, theta.stride(1) if T > 1 else D, M,
        end.data_ptr(), G.data_ptr(), G.stride(1) if T > 1 else D,
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)),
        "rosa_scatter_grad")


def rosa_state_bytes(S: int, K: int, t_capacity: int) -> int:
    return int(load_library().rosa_state_bytes(S, K, t_capacity))


class RosaState:
    """Host handle returned by rosa_build; the caller keeps `buf` alive."""

    def __init__(self, handle, buf):
        self.handle = handle
        self.buf = buf

    def __del__(self):
        try:
            rosa_free(self)
        except Exception:
            pass


def rosa_build(inp: rosa_input, t_capacity: int, state_buf: torch.Tensor,
               out: rosa_out | None = None, stream=None) -> RosaState:
    _require_device(state_buf)
    h = ctypes.c_void_p()
    _check(load_library().rosa_build(
        ctypes.byref(inp), t_capacity, state_buf.data_ptr(),
        state_buf.numel() * state_buf.element_size(), ctypes.byref(h),
        ctypes.byref(out) if out is not None else None, _stream(stream)),
        "rosa_build")
    return RosaState(h, state_buf)


def rosa_step(state: RosaState, row: rosa_input, V, end, sym=None,
              out_row=None, stream=None) -> None:
    """row: one position (T == 1); V: 16-bit [B, Tcap, D] values (position t
    already written) or None; end: int32 [S]; sym: int16 [S] or None;
    out_row: 16-bit [B, D] or None."""
    _require_device(V, end, sym, out_row)
    ldv = V.stride(1) if V is not None else 0
    ldv_b = V.stride(0) if V is not None else 0
    ldo_b = out_row.stride(0) if out_row is not None else 0
    _check(load_library().rosa_step(state.handle, ctypes.byref(row), _ptr(V),
                                    ldv, ldv_b, _ptr(end), _ptr(sym),
                                    _ptr(out_row), ldo_b,
                                    _stream(stream, end.device)),
           "rosa_step")


def rosa_qk_state_bytes(S: int, K: int, t_capacity: int) -> int:
    return int(load_library().rosa_qk_state_bytes(S, K, t_capacity))


def rosa_build_qk(q: rosa_input, k: rosa_input, flags: int, t_capacity: int,
                  state_buf: torch.Tensor, out: rosa_qk_out | None = None,
                  stream=None) -> RosaState:
    """Query/key decode state after the prefix q, k (T may be 0); `out`
    receives the prefix's outputs as rosa_match_qk would."""
    _require_device(state_buf)
    h = ctypes.c_void_p()
    _check(load_library().rosa_build_qk(
        ctypes.byref(q), ctypes.byref(k), flags, t_capacity,
        state_buf.data_ptr(), state_buf.numel() * state_buf.element_size(),
        ctypes.byref(h), ctypes.byref(out) if out is not None else None,
        _stream(stream)), "rosa_build_qk")
    return RosaState(h, state_buf)


def rosa_step_qk(state: RosaState, q_row: rosa_input, k_row: rosa_input,
                 out: rosa_qk_out, stream=None) -> None:
    """One query/key time step for every stream: q_row, k_row with T == 1;
    out: make_qk_out over [S] arrays (cf tables [S, M, 2])."""
    _check(load_library().rosa_step_qk(state.handle, ctypes.byref(q_row),
                                       ctypes.byref(k_row), ctypes.byref(out),
                                       _stream(stream)), "rosa_step_qk")


def rosa_state_length(state: RosaState) -> int:
    return int(load_library().rosa_state_length(state.handle))


def rosa_state_status(state: RosaState, stream=None) -> int:
    return int(load_library().rosa_state_status(state.handle, _stream(stream)))


def rosa_free(state: RosaState) -> None:
    if state.handle:
        load_library().rosa_free(state.handle)
        state.handle = ctypes.c_void_p()


# ------------------------------------------------------------ helpers

def match(x: torch.Tensor, *, K: int | None = None, M: int | None = None,
          want_len: bool = True, want_symbols: bool = False, ws=None,
          stream=None):
    """Allocate outputs (and workspace unless given) with torch and run
    rosa_match.  x: uint8 symbols [S, T] with K, or bf16 [B, T, D] with M.
    Returns (E int32 [S,T], SYM int16 [S,T], L int32 [S,T] or None,
    symbols uint8 [S,T] or None)."""
    if x.dtype == torch.uint8:
        inp = symbols_input(x, K)
        S, T, Kk = x.shape[0], x.shape[1], K
    else:
        inp = bf16_input(x, M)
        B, T, D = x.shape
        S, Kk = B * (D // M), 1 << M
    dev = x.device
    E = torch.empty((S, T), dtype=torch.int32, device=dev)
    SYM = torch.empty((S, T), dtype=torch.int16, device=dev)
    L = torch.empty((S, T), dtype=torch.int32, device=dev) if want_len else None
    syms = (torch.empty((S, T), dtype=torch.uint8, device=dev)
            if want_symbols else None)
    if ws is None:
        ws = torch.empty(rosa_match_workspace_bytes(S, T, Kk), dtype=torch.uint8,
                         device=dev)
    rosa_match(inp, make_out(E, SYM, L, syms), ws, stream)
    return E, SYM, L, syms


def match_qk(q: torch.Tensor, k: torch.Tensor, *, K: int | None = None,
             M: int | None = None, rle: bool = False, cf: bool = False,
             ws=None, stream=None):
    """Allocate outputs (and workspace unless given) and run rosa_match_qk.
    q, k: uint8 symbols [S, T] with K, or bf16 [B, T, D] with M.  Returns a
    dict of int32 tensors: tau, end, len, run_of, run_start, ridx [S, T] and,
    with cf, cf_tau and cf_ridx [S, T, M, 2]."""
    if q.dtype == torch.uint8:
        qi, ki = symbols_input(q, K), symbols_input(k, K)
        S, T, Kk = q.shape[0], q.shape[1], K
        Mm = max(1, (K - 1).bit_length())
    else:
        qi, ki = bf16_input(q, M), bf16_input(k, M)
        B, T, D = q.shape
        S, Kk, Mm = B * (D // M), 1 << M, M
    dev = q.device
    res = {n: torch.empty((S, T), dtype=torch.int32, device=dev)
           for n in ("tau", "end", "len", "run_of", "run_start", "ridx")}
    if cf:
        res["cf_tau"] = torch.empty((S, T, Mm, 2), dtype=torch.int32, device=dev)
        res["cf_ridx"] = torch.empty((S, T, Mm, 2), dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(rosa_match_qk_workspace_bytes(S, T, Kk),
                         dtype=torch.uint8, device=dev)
    out = make_qk_out(res["tau"], **{n: v for n, v in res.items() if n != "tau"})
    rosa_match_qk(qi, ki, ROSA_QK_RLE if rle else 0, out, ws, stream)
    return res
