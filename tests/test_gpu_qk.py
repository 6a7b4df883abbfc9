"""GPU parity of rosa_match_qk (query/key retrieval, run folding,
counterfactual tables) through the C-ABI against the CPU oracle: every
output bit-exact.  Streams cover independent, correlated and equal query and
key streams, long key runs, every alphabet size class, ragged lengths, bf16
inputs and a batched-shaped case."""
import numpy as np
import pytest
import torch

import oracle
from online_suffix_automaton_amd import rosa, synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FIELDS = ("tau", "end", "len", "run_of", "run_start", "ridx")


def _say(msg):
    print(msg, flush=True)


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


def _compare(got, want, what):
    for name, w in want.items():
        g = got[name].cpu().numpy()
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            idx = tuple(bad[0])
            raise AssertionError(f"{what}: {name} differs at {len(bad)} places, "
                                 f"first {idx}: gpu {g[idx]} oracle {w[idx]}")


@pytest.mark.parametrize("K,S,T", [(2, 24, 700), (4, 16, 1500), (16, 40, 2500),
                                   (256, 8, 900), (3, 8, 333)])
@pytest.mark.parametrize("mode", ["same", "indep", "mixed", "runs"])
@pytest.mark.parametrize("rle", [False, True])
def test_qk_symbols(K, S, T, mode, rle):
    _say(f"qk symbols K={K} S={S} T={T} mode={mode} rle={rle}")
    q, k = _streams(1000 + K + T, S, T, K, mode)
    cf = (K & (K - 1)) == 0 and K >= 2
    M = max(1, (K - 1).bit_length())
    got = rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                        K=K, rle=rle, cf=cf)
    torch.cuda.synchronize()
    want = oracle.match_qk(q, k, K, M if cf else 0, rle, cf=cf)
    if not cf:
        want.pop("cf_tau", None)
        want.pop("cf_ridx", None)
    _compare(got, want, f"K={K} {mode} rle={rle}")


def test_qk_equal_streams_match_self_retrieval():
    """q = k without folding: end and len equal rosa_match's E and L."""
    S, T, K = 32, 3000, 16
    x = np.random.default_rng(5).integers(0, K, (S, T)).astype(np.uint8)
    xd = torch.from_numpy(x).to(DEV)
    got = rosa.match_qk(xd, xd, K=K)
    E, _, L, _ = rosa.match(xd, K=K)
    torch.cuda.synchronize()
    assert torch.equal(got["end"], E)
    assert torch.equal(got["len"], L)


@pytest.mark.parametrize("rle", [False, True])
def test_qk_bf16(rle):
    """bf16 hidden states for queries and keys (Sec. 3.2 discretisation on
    the device), M = 4, with counterfactual tables."""
    B, T, D, M = 2, 1200, 64, 4
    Hq = synth.bf16_normal((B, T, D), 21)
    Hk = synth.bf16_normal((B, T, D), 22)
    if rle:   # hold key rows for a few steps so that runs appear
        idx = np.minimum(np.arange(T) // 3 * 3, T - 1)
        Hk = np.ascontiguousarray(Hk[:, idx])
    dq = torch.from_numpy(Hq.view(np.int16)).to(DEV)
    dk = torch.from_numpy(Hk.view(np.int16)).to(DEV)
    got = rosa.match_qk(dq, dk, M=M, rle=rle, cf=True)
    torch.cuda.synchronize()
    q = oracle.discretize_bf16(Hq, M)
    k = oracle.discretize_bf16(Hk, M)
    want = oracle.match_qk(q, k, 1 << M, M, rle, cf=True)
    _compare(got, want, f"bf16 rle={rle}")


@pytest.mark.parametrize("T", [1, 2, 17])
def test_qk_short_streams(T):
    S, K = 5, 4
    q, k = _streams(77 + T, S, T, K, "mixed")
    for rle in (False, True):
        got = rosa.match_qk(torch.from_numpy(q).to(DEV),
                            torch.from_numpy(k).to(DEV), K=K, rle=rle, cf=True)
        torch.cuda.synchronize()
        _compare(got, oracle.match_qk(q, k, K, 2, rle, cf=True), f"T={T}")


def test_qk_symbol_flag():
    S, T, K = 4, 64, 4
    q, k = _streams(3, S, T, K, "indep")
    k[2, 10] = 9
    ws = torch.empty(rosa.rosa_match_qk_workspace_bytes(S, T, K),
                     dtype=torch.uint8, device=DEV)
    rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                  K=K, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_ERR_SYMBOL
    k[2, 10] = 1
    rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                  K=K, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_OK


def test_qk_batched_shape():
    """Batched-workload shape with separate query and key hidden states:
    [8, 4096, 256] bf16, M = 4 (512 streams), folding and counterfactual
    tables on."""
    _say("qk batched shape: generating")
    B, T, D, M = 8, 4096, 256, 4
    Hq = synth.bf16_normal((B, T, D), 31)
    Hk = synth.bf16_normal((B, T, D), 32)
    dq = torch.from_numpy(Hq.view(np.int16)).to(DEV)
    dk = torch.from_numpy(Hk.view(np.int16)).to(DEV)
    _say("gpu")
    got = rosa.match_qk(dq, dk, M=M, rle=True, cf=True)
    torch.cuda.synchronize()
    _say("oracle")
    q = oracle.discretize_bf16(Hq, M)
    k = oracle.discretize_bf16(Hk, M)
    want = oracle.match_qk(q, k, 1 << M, M, True, cf=True)
    _compare(got, want, "batched qk")


@pytest.mark.parametrize("K,T,kind", [(16, 4096, "iid"), (64, 4096, "iid"),
                                      (2, 4096, "iid"), (16, 4096, "const"),
                                      (4, 4096, "period"), (16, 4097, "iid"),
                                      (16, 5000, "period"), (128, 3000, "iid")])
def test_qk_table_placement_limits(K, T, kind):
    """Streams at the largest length and alphabet whose tables live in LDS
    (T = 4096, K = 64), binary streams (most states per step), a constant
    and a periodic key stream (longest suffix paths), and streams just past
    those limits, whose tables live in HBM."""
    S = 3
    _say(f"qk limits K={K} T={T} {kind}")
    rng = np.random.default_rng(4000 + K + T)
    if kind == "iid":
        k = rng.integers(0, K, (S, T))
    elif kind == "const":
        k = np.full((S, T), K - 1)
    else:
        k = np.tile(np.arange(3) % K, T)[: T][None].repeat(S, 0)
    k = k.astype(np.uint8)
    q = np.where(rng.random((S, T)) < 0.8, k, rng.integers(0, K, (S, T))).astype(np.uint8)
    M = (K - 1).bit_length()
    for rle in (False, True):
        got = rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                            K=K, rle=rle, cf=True)
        torch.cuda.synchronize()
        _compare(got, oracle.match_qk(q, k, K, M, rle, cf=True),
                 f"K={K} T={T} {kind} rle={rle}")


def test_qk_many_short_streams():
    """512 streams of 2000 steps: two LDS-resident streams per CU, every
    stream resident at once."""
    S, T, K = 512, 2000, 16
    q, k = _streams(909, S, T, K, "mixed")
    got = rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                        K=K, rle=True, cf=True)
    torch.cuda.synchronize()
    _compare(got, oracle.match_qk(q, k, K, 4, True, cf=True), "512 x 2000")


@pytest.mark.parametrize("rle", [False, True])
def test_qk_long_matches_mixed_with_short(rle):
    """One call mixing streams whose matches grow past 32 units (equal query
    and key streams; query copies of 31, 32, 33 and 40 key units planted at a
    later time) with ordinary independent streams: every stream's outputs,
    whichever kernel answers it, equal the oracle's."""
    S, T, K = 10, 3000, 16
    rng = np.random.default_rng(77 + rle)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    q = rng.integers(0, K, (S, T)).astype(np.uint8)
    q[0] = k[0]
    q[5] = k[5]
    for s, n in ((1, 31), (2, 32), (3, 33), (4, 40), (6, 32), (7, 33)):
        a, b = 100 + 37 * s, 2000 + 11 * s   # key units a..a+n-1 copied to query times b..
        q[s, b:b + n] = k[s, a:a + n]
    _say(f"qk long/short mix rle={rle}")
    got = rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                        K=K, rle=rle, cf=True)
    torch.cuda.synchronize()
    _compare(got, oracle.match_qk(q, k, K, 4, rle, cf=True), f"long/short mix rle={rle}")


@pytest.mark.parametrize("case", range(12))
def test_qk_random_shapes(case):
    """Seeded sweep over the shapes the bit-parallel kernel takes (ragged T
    up to its 4096-unit limit, alphabets 2..64, with and without folding and
    tables, stream counts on both sides of the two-waves-per-stream split),
    each against the oracle."""
    rng = np.random.default_rng(5000 + case)
    K = int(rng.choice([2, 3, 5, 8, 16, 32, 64]))
    T = int(rng.integers(1, 4097))
    S = int(rng.choice([1, 3, 17, 40, 600]))
    if S * T > 600 * 1200:
        T = max(1, (600 * 1200) // S)
    rle = bool(rng.integers(0, 2))
    cf = (K & (K - 1)) == 0 and bool(rng.integers(0, 2))
    mode = ["same", "indep", "mixed", "runs"][int(rng.integers(0, 4))]
    M = (K - 1).bit_length()
    _say(f"qk random case {case}: K={K} T={T} S={S} rle={rle} cf={cf} mode={mode}")
    q, k = _streams(6000 + case, S, T, K, mode)
    got = rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                        K=K, rle=rle, cf=cf)
    torch.cuda.synchronize()
    want = oracle.match_qk(q, k, K, M if cf else 0, rle, cf=cf)
    if not cf:
        want.pop("cf_tau", None)
        want.pop("cf_ridx", None)
    _compare(got, want, f"random case {case}")


@pytest.mark.parametrize("T", [1, 100, 3000, 5000])
@pytest.mark.parametrize("rle", [False, True])
def test_qk_one_symbol(T, rle):
    """A one-symbol alphabet (every stream constant), the shape the grouped
    kernels leave to the bit-parallel kernel (T <= 4096) and the automaton
    (beyond): matches as long as the key history."""
    S = 3
    q = np.zeros((S, T), np.uint8)
    k = np.zeros((S, T), np.uint8)
    _say(f"qk one symbol T={T} rle={rle}")
    got = rosa.match_qk(torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV),
                        K=1, rle=rle)
    torch.cuda.synchronize()
    want = oracle.match_qk(q, k, 1, 0, rle, cf=False)
    want.pop("cf_tau", None)
    want.pop("cf_ridx", None)
    _compare(got, want, f"one symbol T={T} rle={rle}")
