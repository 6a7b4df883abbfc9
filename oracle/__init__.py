"""CPU oracle for ROSA retrieval -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``online_suffix_automaton_amd``) never imports it, and the two share no code.

Source: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
(arXiv 2602.02499).  Each function cites the passage it follows; the
arithmetic lives in ``rosa_oracle.c`` (plain C, built with gcc) apart from
``brute_py``, an independent pure-Python statement of the definition used on
tiny inputs.

All functions take and return numpy arrays on the host:
  * ``discretize_bf16(H_u16 [B,T,D], M) -> sym uint8 [S,T]``   (Sec. 3.2)
  * ``match(sym uint8 [S,T], K) -> (E int32, SYM int16, L int32)``
    (Sec. 2.2, Sec. 3.3 / App. B.3)
  * ``brute(sym [S,T]) -> (E, L)``  O(T^2) definition, pins ``match``
  * ``gather(V_u16 [B,T,D], E [S,T], M) -> out u16 [B,T,D]`` (App. C.4, Eq. 17)
  * ``sam_stats(x [T], K) -> (states, transitions, clones, distinct)``
  * ``match_qk(q [S,T], k [S,T], K, M, rle) -> dict``  query/key retrieval,
    optional run-length folding and per-bit counterfactual destinations
    (Sec. 3.3; App. C.5, C.6; Sec. 4.2 step 3)
  * ``brute_qk_py(q [T], k [T], K, M, rle) -> dict``  the same definition by
    direct search, for tiny streams (pins ``match_qk``)
  * ``scatter_grad(theta f32 [B,T,D], E [S,T], M) -> G f32 [B,T,D]``  the
    transpose of ``gather`` (App. C.4), summed over t in increasing order in
    double precision
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rosa_oracle.c")
# ROSA_ORACLE_LIB selects another build of the same source (the sanitizer
# build of build_sanitized(), loaded by the sanitizer test)
_LIB_PATH = os.environ.get("ROSA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SANITIZED_LIB = os.path.join(_HERE, "liboracle_san.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile rosa_oracle.c with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-shared", "-fPIC",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized() -> str:
    """Compile rosa_oracle.c with AddressSanitizer and UndefinedBehavior-
    Sanitizer (host code only; every UB report aborts) into
    oracle/liboracle_san.so.  A process loads it with the sanitizer runtime
    preloaded and ROSA_ORACLE_LIB pointing at it."""
    tmp = SANITIZED_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-shared", "-fPIC",
                           "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined",
                           "-o", tmp, _SRC])
    os.replace(tmp, SANITIZED_LIB)
    return SANITIZED_LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.oracle_discretize_bf16.argtypes = [P, I64, I64, I64, I, P]
    lib.oracle_match.argtypes = [P, I64, I, P, P, P]
    lib.oracle_match_streams.argtypes = [P, I64, I64, I64, I, P, P, P]
    lib.oracle_sam_stats.argtypes = [P, I64, I, P]
    lib.oracle_brute.argtypes = [P, I64, P, P]
    lib.oracle_gather.argtypes = [P, I64, I64, I64, I, P, P]
    lib.oracle_match_qk.argtypes = [P, P, I64, I, I, I] + [P] * 8
    lib.oracle_scatter_grad.argtypes = [P, I64, I64, I64, I, P, P]
    for f in (lib.oracle_discretize_bf16, lib.oracle_match,
              lib.oracle_match_streams, lib.oracle_sam_stats,
              lib.oracle_brute, lib.oracle_gather, lib.oracle_match_qk,
              lib.oracle_scatter_grad):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc == -2:
        raise ValueError(f"{what}: symbol out of range [0, K)")
    if rc != 0:
        raise ValueError(f"{what}: error code {rc}")


def discretize_bf16(H: np.ndarray, M: int) -> np.ndarray:
    """Sec. 3.2, Eq. (10)-(15): bit = I[h > 0] per channel, route r packs
    channels r*M .. r*M+M-1 with weight 2^j.  H: uint16 bf16 bits [B,T,D]."""
    H = np.ascontiguousarray(H, dtype=np.uint16)
    B, T, D = H.shape
    S = B * (D // M)
    sym = np.zeros((S, T), dtype=np.uint8)
    _check(_load().oracle_discretize_bf16(_ptr(H), B, T, D, M, _ptr(sym)),
           "discretize")
    return sym


def match(sym: np.ndarray, K: int):
    """Sec. 2.2 + Sec. 3.3: per stream, longest recurring suffix, its most
    recent earlier end E (-1 if none) and the next symbol x[E+1]."""
    sym = np.ascontiguousarray(sym, dtype=np.uint8)
    if sym.ndim == 1:
        sym = sym[None, :]
    S, T = sym.shape
    E = np.empty((S, T), dtype=np.int32)
    SYM = np.empty((S, T), dtype=np.int16)
    L = np.empty((S, T), dtype=np.int32)
    _check(_load().oracle_match_streams(_ptr(sym), S, T, T, K, _ptr(E),
                                        _ptr(SYM), _ptr(L)), "match")
    return E, SYM, L


def match_one(x: np.ndarray, K: int, E: np.ndarray, SYM: np.ndarray,
              L: np.ndarray) -> None:
    """One stream into caller-provided rows (used by threaded baselines)."""
    _check(_load().oracle_match(_ptr(x), x.shape[0], K, _ptr(E), _ptr(SYM),
                                _ptr(L)), "match")


def brute(sym: np.ndarray):
    """The definition as an O(T^2) common-suffix table (pins ``match``)."""
    sym = np.ascontiguousarray(sym, dtype=np.uint8)
    if sym.ndim == 1:
        sym = sym[None, :]
    S, T = sym.shape
    E = np.empty((S, T), dtype=np.int32)
    L = np.empty((S, T), dtype=np.int32)
    lib = _load()
    for s in range(S):
        row = np.ascontiguousarray(sym[s])
        e = np.empty(T, dtype=np.int32)
        l = np.empty(T, dtype=np.int32)
        _check(lib.oracle_brute(_ptr(row), T, _ptr(e), _ptr(l)), "brute")
        E[s], L[s] = e, l
    return E, L


def brute_py(x):
    """Pure-Python restatement of the definition for tiny streams: for each
    t, scan every earlier end e, count the common suffix length directly, keep
    the longest and, among equals, the latest."""
    x = [int(v) for v in x]
    T = len(x)
    E, L = [], []
    for t in range(T):
        best, arg = 0, -1
        for e in range(t):
            k = 0
            while e - k >= 0 and x[e - k] == x[t - k]:
                k += 1
            if k > 0 and k >= best:
                best, arg = k, e
        E.append(arg)
        L.append(best)
    return E, L


def gather(V: np.ndarray, E: np.ndarray, M: int) -> np.ndarray:
    """App. C.4: read-out at tau = E+1 for the route's M channels; zero when
    there is no hit (validity mask, Eq. (17))."""
    V = np.ascontiguousarray(V, dtype=np.uint16)
    B, T, D = V.shape
    E = np.ascontiguousarray(E, dtype=np.int32)
    out = np.empty_like(V)
    _check(_load().oracle_gather(_ptr(V), B, T, D, M, _ptr(E), _ptr(out)),
           "gather")
    return out


def sam_stats(x: np.ndarray, K: int):
    """(states, transitions, clones, distinct substrings) of the automaton."""
    x = np.ascontiguousarray(x, dtype=np.uint8)
    out = np.zeros(4, dtype=np.int64)
    _check(_load().oracle_sam_stats(_ptr(x), x.shape[0], K, _ptr(out)),
           "sam_stats")
    return tuple(int(v) for v in out)


QK_FIELDS = ("tau", "end", "len", "run_of", "run_start", "ridx")


def match_qk(q: np.ndarray, k: np.ndarray, K: int, M: int = 0,
             rle: bool = False, cf: bool = False):
    """Query/key retrieval (Sec. 3.3): per time t the destination tau of the
    longest suffix of the query units that occurs in the earlier key units,
    its most recent end unit ``end`` and length ``len``; with ``rle`` the
    key stream is folded into runs (``run_of``, ``run_start``, ``ridx``);
    with ``cf`` the per-bit counterfactual tables ``cf_tau``/``cf_ridx``
    [S,T,M,2] (App. C.5, C.6).  q, k: uint8 [S,T] (or [T])."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    if q.ndim == 1:
        q, k = q[None, :], k[None, :]
    S, T = q.shape
    out = {f: np.empty((S, T), np.int32) for f in QK_FIELDS}
    if cf:
        out["cf_tau"] = np.empty((S, T, M, 2), np.int32)
        out["cf_ridx"] = np.empty((S, T, M, 2), np.int32)
    lib = _load()
    for s_ in range(S):
        rows = {f: np.empty(T, np.int32) for f in QK_FIELDS}
        cft = np.empty((T, M, 2), np.int32) if cf else None
        cfr = np.empty((T, M, 2), np.int32) if cf else None
        qs, ks = np.ascontiguousarray(q[s_]), np.ascontiguousarray(k[s_])
        _check(lib.oracle_match_qk(_ptr(qs), _ptr(ks), T, K, M, int(rle),
                                   *[_ptr(rows[f]) for f in QK_FIELDS],
                                   _ptr(cft) if cf else None,
                                   _ptr(cfr) if cf else None), "match_qk")
        for f in QK_FIELDS:
            out[f][s_] = rows[f]
        if cf:
            out["cf_tau"][s_], out["cf_ridx"][s_] = cft, cfr
    return out


def brute_qk_py(q, k, K: int, M: int = 0, rle: bool = False):
    """The query/key definition by direct search, pure Python, tiny streams.
    Units as in ``match_qk``; at unit u every earlier key unit e is scanned,
    the common suffix of Q[..u] and C[..e] counted symbol by symbol, the
    longest kept and among equals the latest; the destination time is the
    start of unit e+1 when it exists and is before t.  Counterfactuals
    replace Q[u] by the symbol with bit j forced to v."""
    q = [int(v) for v in q]
    k = [int(v) for v in k]
    T = len(q)
    start, unit = [], []
    for t in range(T):
        if not rle or t == 0 or k[t] != k[t - 1]:
            start.append(t)
        unit.append(len(start) - 1)
    N = len(start)
    C = [k[s] for s in start]
    Q = [q[s] for s in start]

    def best(u, qu):
        b, arg = 0, -1
        for e in range(u):
            n = 0
            while e - n >= 0 and u - n >= 0:
                a = qu if n == 0 else Q[u - n]
                if a != C[e - n]:
                    break
                n += 1
            if n > 0 and n >= b:
                b, arg = n, e
        return b, arg

    def dest(e, t):
        if e < 0 or e + 1 >= N:
            return -1
        return start[e + 1] if start[e + 1] < t else -1

    res = {f: [] for f in QK_FIELDS}
    res["cf_tau"], res["cf_ridx"] = [], []
    per_unit = [best(u, Q[u]) for u in range(N)]
    cfu = [[[best(u, (Q[u] & ~(1 << j)) | (v << j))[1] for v in (0, 1)]
            for j in range(M)] for u in range(N)]
    for t in range(T):
        u = unit[t]
        ln, e = per_unit[u]
        tt = dest(e, t)
        res["tau"].append(tt)
        res["end"].append(e)
        res["len"].append(ln)
        res["run_of"].append(u)
        res["run_start"].append(start[t] if t < N else -1)
        res["ridx"].append(e + 1 if tt >= 0 else -1)
        res["cf_tau"].append([[dest(cfu[u][j][v], t) for v in (0, 1)]
                              for j in range(M)])
        res["cf_ridx"].append([[cfu[u][j][v] + 1 if dest(cfu[u][j][v], t) >= 0
                                else -1 for v in (0, 1)] for j in range(M)])
    return res


def scatter_grad(theta: np.ndarray, E: np.ndarray, M: int) -> np.ndarray:
    """App. C.4: G[b, tau, c] = sum_t theta[b, t, c] * [E[s, t] + 1 == tau]
    (s = b*R + c // M; E < 0 adds nothing), the transpose of ``gather``.
    theta: float32 [B, T, D]."""
    theta = np.ascontiguousarray(theta, dtype=np.float32)
    B, T, D = theta.shape
    E = np.ascontiguousarray(E, dtype=np.int32)
    G = np.empty_like(theta)
    _check(_load().oracle_scatter_grad(_ptr(theta), B, T, D, M, _ptr(E),
                                       _ptr(G)), "scatter_grad")
    return G
