"""Seeded synthetic inputs for ROSA retrieval.

This module only draws inputs; it holds none of the retrieval arithmetic, and
both the GPU path's tests/bench and the CPU oracle's tests read the same
arrays from it.  Random numbers come from numpy's PCG64 ``default_rng(seed)``.
bf16 tensors are float32 N(0,1) rounded to nearest-even by torch on the CPU
and returned as their uint16 bit patterns.

The paper's workloads (Qwen3 hidden states on LongBench / PG19 / MQAR) are not
available; these stand in for them with the shapes of the five workloads:

  tiny     4 streams, T=256, binary i.i.d. symbols                   (seed 1)
  batched  H [8, 4096, 256] bf16 N(0,1), M=4  -> 512 streams, K=16    (seed 2)
  repeat   1024 streams, T=32768, K=16, i.i.d. base with planted
           copies of earlier spans (length U{32..512}), ~30% coverage (3+s)
  long     H [1, 65536, 2048] bf16 N(0,1), M=4 -> 512 streams, K=16
           plus V [1, 65536, 2048] bf16 N(0,1)                    (seeds 4, 44)
  decode   the long workload as prefix plus 1024 appended rows of H and V
                                                                 (seeds 5, 55)
"""
from __future__ import annotations

import numpy as np


def bf16_normal(shape, seed: int, chunk_rows: int = 4096) -> np.ndarray:
    """float32 N(0,1) rounded to bf16 (RNE), as uint16 bit patterns."""
    import torch

    rng = np.random.default_rng(seed)
    shape = tuple(int(v) for v in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1])
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        f = rng.standard_normal((r1 - r0, shape[-1]), dtype=np.float32)
        t = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16)
        flat[r0:r1] = t.numpy().view(np.uint16)
    return out


def iid_symbols(S: int, T: int, K: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(0, K, size=(S, T), dtype=np.uint8)


def planted_copies(T: int, K: int, seed: int, gap_mean: float = 635.0,
                   len_lo: int = 32, len_hi: int = 512) -> np.ndarray:
    """i.i.d. base; then left to right: skip a geometric gap, copy an earlier,
    non-overlapping span of length U{len_lo..len_hi} (clipped at T) over the
    current position.  Sources may contain earlier copies."""
    rng = np.random.default_rng(seed)
    x = rng.integers(0, K, size=T, dtype=np.uint8)
    t = 0
    while True:
        t += int(rng.geometric(1.0 / gap_mean))
        if t >= T:
            break
        ln = int(rng.integers(len_lo, len_hi + 1))
        ln = min(ln, T - t)
        if ln <= 0 or t - ln < 0:
            t += max(ln, 1)
            continue
        src = int(rng.integers(0, t - ln + 1))
        x[t:t + ln] = x[src:src + ln]
        t += ln
    return x


def repeat_streams(S: int = 1024, T: int = 32768, K: int = 16,
                   seed0: int = 3) -> np.ndarray:
    return np.stack([planted_copies(T, K, seed0 + s) for s in range(S)])


# ---------------------------------------------------------------- workloads

def tiny():
    return {"kind": "symbols", "sym": iid_symbols(4, 256, 2, 1), "K": 2}


def batched():
    return {"kind": "bf16", "H": bf16_normal((8, 4096, 256), 2), "M": 4}


def repeat(S: int = 1024, T: int = 32768):
    return {"kind": "symbols", "sym": repeat_streams(S, T, 16, 3), "K": 16}


def long(T: int = 65536, D: int = 2048, with_v: bool = True):
    w = {"kind": "bf16", "H": bf16_normal((1, T, D), 4), "M": 4}
    if with_v:
        w["V"] = bf16_normal((1, T, D), 44)
    return w


def decode_tail(n: int = 1024, D: int = 2048):
    """Rows appended after the long workload's prefix."""
    return {"H": bf16_normal((1, n, D), 5), "V": bf16_normal((1, n, D), 55)}


# ------------------------------------------------------ structured streams

def constant(T: int, c: int = 0) -> np.ndarray:
    return np.full(T, c, dtype=np.uint8)


def periodic(T: int, pattern) -> np.ndarray:
    p = np.asarray(pattern, dtype=np.uint8)
    return np.resize(p, T).astype(np.uint8)


def fibonacci_word(T: int) -> np.ndarray:
    a, b = [0], [0, 1]
    while len(b) < T:
        a, b = b, b + a
    return np.asarray(b[:T], dtype=np.uint8)


def de_bruijn(K: int, n: int) -> np.ndarray:
    """Lexicographically least de Bruijn sequence B(K, n) (FKM algorithm)."""
    a = [0] * (K * n)
    seq = []

    def db(t, p):
        if t > n:
            if n % p == 0:
                seq.extend(a[1:p + 1])
        else:
            a[t] = a[t - p]
            db(t + 1, p)
            for j in range(a[t - p] + 1, K):
                a[t] = j
                db(t + 1, t)

    db(1, 1)
    return np.asarray(seq, dtype=np.uint8)


def onehot_bf16(B: int, T: int, D: int, positive_channels, value=0x3F80):
    """All zero except the listed (b, t, c) entries set to ``value``."""
    H = np.zeros((B, T, D), dtype=np.uint16)
    for (b, t, c) in positive_channels:
        H[b, t, c] = value
    return H
