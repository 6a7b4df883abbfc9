"""Pins for the query/key oracle (no GPU): hand-worked examples
(tests/golden/qk_examples.json), an independent pure-Python direct search of
the definition on many tiny streams (with and without run folding and
counterfactual tables), reduction to the self-match oracle when q = k, and
invariants of folding and of the counterfactual tables."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
EXAMPLES = json.load(open(os.path.join(GOLD, "qk_examples.json")))["examples"]


@pytest.mark.parametrize("ex", EXAMPLES, ids=lambda e: e["name"])
def test_qk_hand_examples(ex):
    q = np.asarray(ex["q"], np.uint8)
    k = np.asarray(ex["k"], np.uint8)
    cf = "cf_tau" in ex
    o = oracle.match_qk(q, k, ex["K"], ex["M"], ex["rle"], cf=cf)
    for f in ("tau", "end", "len", "run_of", "run_start", "ridx"):
        if f in ex:
            assert o[f][0].tolist() == ex[f], f
    if cf:
        assert o["cf_tau"][0].tolist() == ex["cf_tau"]
    b = oracle.brute_qk_py(q, k, ex["K"], ex["M"], ex["rle"])
    for f in ("tau", "end", "len"):
        assert b[f] == ex[f], f
    if cf:
        assert b["cf_tau"] == ex["cf_tau"]


def _streams(rng, T, K, mode):
    k = rng.integers(0, K, T).astype(np.uint8)
    if mode == "same":
        q = k.copy()
    elif mode == "indep":
        q = rng.integers(0, K, T).astype(np.uint8)
    elif mode == "mixed":
        q = np.where(rng.random(T) < 0.7, k,
                     rng.integers(0, K, T)).astype(np.uint8)
    else:  # runs: long runs of equal key symbols
        k = np.repeat(rng.integers(0, K, T), rng.integers(1, 5, T))[:T]
        k = k.astype(np.uint8)
        q = np.where(rng.random(T) < 0.5, k,
                     rng.integers(0, K, T)).astype(np.uint8)
    return q, k


@pytest.mark.parametrize("rle", [False, True])
@pytest.mark.parametrize("mode", ["same", "indep", "mixed", "runs"])
def test_qk_against_direct_search(rle, mode):
    rng = np.random.default_rng(100 + 10 * rle + len(mode))
    for _ in range(60):
        T = int(rng.integers(1, 48))
        M = int(rng.integers(1, 4))
        K = 1 << M
        q, k = _streams(rng, T, K, mode)
        o = oracle.match_qk(q, k, K, M, rle, cf=True)
        b = oracle.brute_qk_py(q, k, K, M, rle)
        for f in oracle.QK_FIELDS:
            assert o[f][0].tolist() == b[f], (f, T, M)
        assert o["cf_tau"][0].tolist() == b["cf_tau"]
        assert o["cf_ridx"][0].tolist() == b["cf_ridx"]


def test_qk_reduces_to_self_match():
    """q = k without folding is the self-match definition (same L and E);
    tau keeps E+1 only when it is before t."""
    rng = np.random.default_rng(7)
    for K, T in [(2, 3000), (16, 5000), (256, 2000)]:
        x = rng.integers(0, K, T).astype(np.uint8)
        o = oracle.match_qk(x, x, K)
        E, _, L = oracle.match(x, K)
        assert np.array_equal(o["end"][0], E[0])
        assert np.array_equal(o["len"][0], L[0])
        t = np.arange(T)
        want = np.where((E[0] >= 0) & (E[0] + 1 < t), E[0] + 1, -1)
        assert np.array_equal(o["tau"][0], want)


def test_rle_without_repeats_is_plain():
    """Folding changes nothing when no two adjacent key symbols are equal."""
    rng = np.random.default_rng(8)
    T, K = 3000, 16
    k = np.empty(T, np.uint8)
    k[0] = 3
    for t in range(1, T):
        k[t] = (k[t - 1] + rng.integers(1, K)) % K
    q = rng.integers(0, K, T).astype(np.uint8)
    a = oracle.match_qk(q, k, K, 4, False, cf=True)
    b = oracle.match_qk(q, k, K, 4, True, cf=True)
    for f in ("tau", "end", "len", "cf_tau"):
        assert np.array_equal(a[f], b[f]), f
    assert np.array_equal(b["run_of"][0], np.arange(T))
    assert np.array_equal(b["run_start"][0], np.arange(T))


def test_rle_runs_and_destinations():
    """Invariants at a larger size: run starts are the positions where the
    key symbol changes; tau is the start of a run, before t; with q = k the
    destination run is never the current one."""
    rng = np.random.default_rng(9)
    T, K = 20000, 4
    k = np.repeat(rng.integers(0, K, T), rng.integers(1, 6, T))[:T].astype(np.uint8)
    o = oracle.match_qk(k, k, K, 2, True, cf=True)
    starts = np.flatnonzero(np.r_[True, k[1:] != k[:-1]])
    N = len(starts)
    assert np.array_equal(o["run_start"][0][:N], starts)
    assert np.all(o["run_start"][0][N:] == -1)
    assert np.array_equal(o["run_of"][0], np.cumsum(np.r_[True, k[1:] != k[:-1]]) - 1)
    tau, ridx, t = o["tau"][0], o["ridx"][0], np.arange(T)
    v = tau >= 0
    assert np.all(tau[v] < t[v])
    assert np.array_equal(starts[ridx[v]], tau[v])
    assert np.all(ridx[v] < o["run_of"][0][v])
    assert np.all(ridx[~v] == -1)


def test_counterfactual_actual_bit_is_the_forward_pass():
    """Forcing a bit to the value it already has reproduces tau (App. C.5:
    one of the two branches is the true forward pass)."""
    rng = np.random.default_rng(10)
    T, M = 4000, 4
    K = 1 << M
    for rle in (False, True):
        k = np.repeat(rng.integers(0, K, T), rng.integers(1, 3, T))[:T].astype(np.uint8)
        q = np.where(rng.random(T) < 0.6, k, rng.integers(0, K, T)).astype(np.uint8)
        o = oracle.match_qk(q, k, K, M, rle, cf=True)
        starts = np.flatnonzero(np.r_[True, k[1:] != k[:-1]]) if rle else np.arange(T)
        qu = q[starts][o["run_of"][0]] if rle else q
        for j in range(M):
            bit = (qu >> j) & 1
            got = np.take_along_axis(o["cf_tau"][0][:, j, :], bit[:, None].astype(np.int64), 1)[:, 0]
            assert np.array_equal(got, o["tau"][0])
