"""GPU parity of rosa_match_qk on streams of more than 4096 steps: the
grouped-key kernels (keys sorted by their last d symbols, one thread per
query unit), with the time-ordered pass answering the query symbols they
leave (key groups past their cap, matches running more than 1024 units past
d).  Every output is compared bit-exact with the CPU oracle: independent,
correlated and equal query and key streams, key runs, alphabets 2..256
(powers of two with the counterfactual tables, 3 without), ragged lengths,
low-entropy streams up to 65536 steps, planted long matches and the
64 x 65536 bf16 shape."""
import concurrent.futures as cf_pool
import os

import numpy as np
import pytest
import torch

import oracle
from online_suffix_automaton_amd import rosa, synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _oracle(q, k, K, M, rle, cf):
    """oracle.match_qk over the streams, split across threads at stream
    boundaries (the library call releases the interpreter lock)."""
    S = q.shape[0]
    n = max(1, min(16, os.cpu_count() or 1, S))
    parts = [c for c in np.array_split(np.arange(S), n) if len(c)]

    def one(c):
        return oracle.match_qk(q[c[0]:c[-1] + 1], k[c[0]:c[-1] + 1], K, M, rle, cf=cf)

    with cf_pool.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        outs = list(ex.map(one, parts))
    return {name: np.concatenate([o[name] for o in outs]) for name in outs[0]}


def _compare(got, want, what):
    for name, w in want.items():
        g = got[name].cpu().numpy()
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            idx = tuple(bad[0])
            raise AssertionError(f"{what}: {name} differs at {len(bad)} places, "
                                 f"first {idx}: gpu {g[idx]} oracle {w[idx]}")


def _run(q, k, K, rle, cf, what):
    M = max(1, (K - 1).bit_length())
    _say(what)
    got = rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                        K=K, rle=rle, cf=cf)
    torch.cuda.synchronize()
    want = _oracle(q, k, K, M if cf else 0, rle, cf)
    if not cf:
        want.pop("cf_tau", None)
        want.pop("cf_ridx", None)
    _compare(got, want, what)


def _streams(seed, S, T, K, mode):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    if mode == "runs":
        k = np.stack([np.repeat(rng.integers(0, K, T), rng.integers(1, 6, T))[:T]
                      for _ in range(S)]).astype(np.uint8)
    if mode == "same":
        q = k.copy()
    elif mode == "indep":
        q = rng.integers(0, K, (S, T)).astype(np.uint8)
    else:
        q = np.where(rng.random((S, T)) < 0.7, k,
                     rng.integers(0, K, (S, T))).astype(np.uint8)
    return q, k


@pytest.mark.parametrize("K", [2, 3, 4, 16, 64, 256])
@pytest.mark.parametrize("mode", ["same", "indep", "mixed", "runs"])
@pytest.mark.parametrize("rle", [False, True])
def test_qk_grouped_symbols(K, mode, rle):
    """5 streams of 9001 steps (not a multiple of a chunk, a query
    workgroup or a segment) for every alphabet class and stream relation."""
    S, T = 5, 9001
    q, k = _streams(7000 + K, S, T, K, mode)
    cf = (K & (K - 1)) == 0
    _run(q, k, K, rle, cf, f"grouped K={K} mode={mode} rle={rle}")


@pytest.mark.parametrize("rle", [False, True])
def test_qk_grouped_bf16_64x65536(rle):
    """The long-context shape: query and key hidden states [1, 65536, 256]
    bf16, M = 4 (64 streams of 65536 steps, K = 16), with the
    counterfactual tables."""
    B, T, D, M = 1, 65536, 256, 4
    Hq = synth.bf16_normal((B, T, D), 41)
    Hk = synth.bf16_normal((B, T, D), 42)
    dq = torch.from_numpy(Hq.view(np.int16)).to(DEV)
    dk = torch.from_numpy(Hk.view(np.int16)).to(DEV)
    _say(f"grouped bf16 64 x 65536 rle={rle}")
    got = rosa.match_qk(dq, dk, M=M, rle=rle, cf=True)
    torch.cuda.synchronize()
    q = oracle.discretize_bf16(Hq, M)
    k = oracle.discretize_bf16(Hk, M)
    _compare(got, _oracle(q, k, 1 << M, M, rle, True), f"bf16 64x65536 rle={rle}")


@pytest.mark.parametrize("rle", [False, True])
def test_qk_grouped_low_entropy(rle):
    """Streams the groups cannot hold or that repeat for long: constant key
    and query streams, a dead query channel, periodic streams (period 3 and
    a period-7 pattern with rare noise), next to ordinary streams in the same
    call.  Whichever kernel answers a stream, its outputs equal the
    oracle's."""
    S, T, K = 8, 20000, 16
    rng = np.random.default_rng(91 + rle)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    q = rng.integers(0, K, (S, T)).astype(np.uint8)
    k[0] = 5                                   # constant key stream
    q[1] = 3                                   # dead query channel
    k[2] = 7
    q[2] = 7                                   # both constant, equal
    k[3] = np.tile([1, 2, 3], T)[:T]           # period 3
    q[3] = k[3]
    pat = rng.integers(0, K, 7)
    k[4] = np.tile(pat, T)[:T]
    noise = rng.random(T) < 0.001
    k[4, noise] = rng.integers(0, K, int(noise.sum()))
    q[4] = np.tile(pat, T)[:T]
    _run(q, k, K, rle, True, f"grouped low entropy rle={rle}")


@pytest.mark.parametrize("rle", [False, True])
def test_qk_grouped_long_matches(rle):
    """Query copies of 20, 100, 900, 1100 and 3000 key units planted later
    in the stream (the last two run past the 1024-unit extension limit), and
    equal query and key streams, beside independent streams."""
    S, T, K = 7, 12000, 16
    rng = np.random.default_rng(55 + rle)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    q = rng.integers(0, K, (S, T)).astype(np.uint8)
    for s, n in ((0, 20), (1, 100), (2, 900), (3, 1100), (4, 3000)):
        a, b = 200 + 13 * s, 6000 + 17 * s
        q[s, b:b + n] = k[s, a:a + n]
    q[5] = k[5]
    _run(q, k, K, rle, True, f"grouped long matches rle={rle}")


@pytest.mark.parametrize("case", range(10))
def test_qk_grouped_random_shapes(case):
    """Seeded sweep past the bit-parallel limit: ragged lengths 4097..30000,
    alphabets 2..256, stream counts on both sides of the eight-XCD stream
    mapping, with and without folding and tables."""
    rng = np.random.default_rng(8100 + case)
    K = int(rng.choice([2, 3, 5, 8, 16, 32, 64, 128, 256]))
    T = int(rng.integers(4097, 30001))
    S = int(rng.choice([1, 3, 8, 9, 20]))
    rle = bool(rng.integers(0, 2))
    cf = (K & (K - 1)) == 0 and bool(rng.integers(0, 2))
    mode = ["same", "indep", "mixed", "runs"][int(rng.integers(0, 4))]
    q, k = _streams(8200 + case, S, T, K, mode)
    _run(q, k, K, rle, cf,
         f"grouped random case {case}: K={K} T={T} S={S} rle={rle} cf={cf} mode={mode}")


@pytest.mark.parametrize("rle", [False, True])
def test_qk_grouped_low_entropy_65536(rle):
    """The time-ordered pass at the long-context length: a constant key
    stream under a random query, equal constant streams, equal period-3
    streams, a period-5 pattern with a repeated symbol (counterfactual
    symbols match the pattern shifted, long past the groups' limit), a
    period-7 key stream with rare noise under its clean query, and an
    independent pair."""
    S, T, K = 6, 65536, 16
    rng = np.random.default_rng(4242 + rle)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    q = rng.integers(0, K, (S, T)).astype(np.uint8)
    k[0] = 9
    k[1] = 4
    q[1] = 4
    k[2] = np.tile([1, 2, 3], T)[:T]
    q[2] = k[2]
    k[3] = np.tile([6, 6, 2, 11, 2], T)[:T]
    q[3] = k[3]
    pat = rng.integers(0, K, 7)
    k[4] = np.tile(pat, T)[:T]
    noise = rng.random(T) < 0.0005
    k[4, noise] = rng.integers(0, K, int(noise.sum()))
    q[4] = np.tile(pat, T)[:T]
    _run(q, k, K, rle, True, f"grouped low entropy 65536 rle={rle}")
