"""GPU parity of the query/key decode: rosa_build_qk over a prefix, then one
rosa_step_qk per time step.  The prefix's outputs and every step's outputs
are compared bit-exact with the oracle's query/key match over the whole
streams; its per-time outputs depend only on q and k up to that time, so
they are what an online decoder must produce.  Symbol and bf16 inputs, with
and without run folding and counterfactual tables, on independent,
correlated, constant and periodic streams, an empty prefix and a prefix
that ends inside a key run; plus the handle's error paths."""
import numpy as np
import pytest
import torch

import oracle
from online_suffix_automaton_amd import rosa, synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
FIELDS = ("tau", "end", "len", "run_of", "ridx")


def _say(msg):
    print(msg, flush=True)


def _decode(qin_at, kin_at, S, T, K, T0, rle, M):
    """Build over times [0, T0) and step through [T0, T).  qin_at(a, b) and
    kin_at(a, b) give rosa_inputs over times [a, b).  Returns the outputs as
    numpy [S, T] arrays (cf tables [S, T, M, 2]) and the prefix run_start."""
    cf = M > 0
    buf = torch.empty(rosa.rosa_qk_state_bytes(S, K, T), dtype=torch.uint8,
                      device=DEV)
    flags = rosa.ROSA_QK_RLE if rle else 0
    pre = {f: torch.full((S, T0), -7, dtype=torch.int32, device=DEV) for f in FIELDS}
    pre["run_start"] = torch.full((S, T0), -7, dtype=torch.int32, device=DEV)
    if cf:
        for f in ("cf_tau", "cf_ridx"):
            pre[f] = torch.full((S, T0, M, 2), -7, dtype=torch.int32, device=DEV)
    out = rosa.make_qk_out(pre["tau"], **{f: v for f, v in pre.items() if f != "tau"})
    h = rosa.rosa_build_qk(qin_at(0, T0), kin_at(0, T0), flags, T, buf, out)
    # steps: outputs of step t in row t of [T, S] buffers (contiguous [S])
    stp = {f: torch.full((T, S), -7, dtype=torch.int32, device=DEV) for f in FIELDS}
    if cf:
        for f in ("cf_tau", "cf_ridx"):
            stp[f] = torch.full((T, S, M, 2), -7, dtype=torch.int32, device=DEV)
    for t in range(T0, T):
        o = rosa.make_qk_out(stp["tau"][t], **{f: v[t] for f, v in stp.items() if f != "tau"})
        rosa.rosa_step_qk(h, qin_at(t, t + 1), kin_at(t, t + 1), o)
    assert rosa.rosa_state_length(h) == T
    assert rosa.rosa_state_status(h) == rosa.ROSA_OK
    got = {}
    for f in FIELDS + (("cf_tau", "cf_ridx") if cf else ()):
        a = stp[f].cpu().numpy()
        a = np.moveaxis(a, 0, 1).copy()          # [S, T, ...]
        if T0 > 0:
            a[:, :T0] = pre[f].cpu().numpy()
        got[f] = a
    rosa.rosa_free(h)
    return got, pre["run_start"].cpu().numpy()


def _check(got, rs, want, T0, what):
    for f, w in want.items():
        if f == "run_start":
            continue
        g = got[f]
        if not np.array_equal(g, w):
            bad = np.argwhere(g != w)
            i = tuple(bad[0])
            raise AssertionError(f"{what}: {f} differs at {len(bad)} places, first "
                                 f"{i}: gpu {g[i]} oracle {w[i]}")
    if T0 > 0:
        # the prefix's run starts: units that began before T0, then -1
        last = want["run_of"][:, T0 - 1]
        exp = np.where(np.arange(T0)[None, :] <= last[:, None],
                       want["run_start"][:, :T0], -1)
        assert np.array_equal(rs, exp), f"{what}: prefix run_start"


def _symbols_case(q, k, K, T0, rle, what):
    S, T = q.shape
    M = (K.bit_length() - 1) if K >= 2 and (K & (K - 1)) == 0 else 0
    qd, kd = torch.from_numpy(q).to(DEV), torch.from_numpy(k).to(DEV)
    _say(what)
    got, rs = _decode(lambda a, b: rosa.symbols_input(qd[:, a:b], K),
                      lambda a, b: rosa.symbols_input(kd[:, a:b], K),
                      S, T, K, T0, rle, M)
    want = oracle.match_qk(q, k, K, M, rle, cf=M > 0)
    _check(got, rs, want, T0, what)


def _streams(seed, S, T, K, mode):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    if mode == "runs":
        k = np.stack([np.repeat(rng.integers(0, K, T), rng.integers(1, 5, T))[:T]
                      for _ in range(S)]).astype(np.uint8)
    if mode == "same":
        q = k.copy()
    elif mode == "indep":
        q = rng.integers(0, K, (S, T)).astype(np.uint8)
    else:
        q = np.where(rng.random((S, T)) < 0.7, k,
                     rng.integers(0, K, (S, T))).astype(np.uint8)
    return q, k


@pytest.mark.parametrize("rle", [False, True])
@pytest.mark.parametrize("K,T0", [(16, 0), (16, 257), (2, 1), (3, 100), (1, 40),
                                  (256, 64)])
def test_qk_decode_symbols(K, T0, rle):
    """Every alphabet class (power of two with tables, 3 without, one
    symbol), prefixes from empty to several hundred steps."""
    S, T = 5, 480
    for mode in ("mixed", "runs"):
        q, k = _streams(300 + K + T0 + rle, S, T, K, mode)
        _symbols_case(q, k, K, T0, rle, f"qk decode K={K} T0={T0} rle={rle} {mode}")


@pytest.mark.parametrize("rle", [False, True])
def test_qk_decode_low_entropy(rle):
    """Constant key stream under a random query, equal constant streams,
    equal period-3 streams, a period-5 pattern with a repeated symbol and a
    key run that spans the end of the prefix."""
    S, T, K, T0 = 5, 400, 16, 150
    rng = np.random.default_rng(77 + rle)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    q = rng.integers(0, K, (S, T)).astype(np.uint8)
    k[0] = 9
    k[1] = 4
    q[1] = 4
    k[2] = np.tile([1, 2, 3], T)[:T]
    q[2] = k[2]
    k[3] = np.tile([6, 6, 2, 11, 2], T)[:T]
    q[3] = k[3]
    k[4, 140:170] = 5                      # a run across the prefix's end
    _symbols_case(q, k, K, T0, rle, f"qk decode low entropy rle={rle}")


@pytest.mark.parametrize("rle", [False, True])
def test_qk_decode_bf16(rle):
    """bf16 query and key hidden states [2, 300, 32], M = 4 (16 streams),
    prefix of 120 steps, then one row per step."""
    B, T, D, M, T0 = 2, 300, 32, 4, 120
    Hq = synth.bf16_normal((B, T, D), 61)
    Hk = synth.bf16_normal((B, T, D), 62)
    # correlated rows: the query copies the key at most positions
    sel = np.random.default_rng(63).random((B, T)) < 0.6
    Hq[sel] = Hk[sel]
    hq = torch.from_numpy(Hq.view(np.int16)).to(DEV)
    hk = torch.from_numpy(Hk.view(np.int16)).to(DEV)
    S, K = B * D // M, 1 << M
    _say(f"qk decode bf16 rle={rle}")
    got, rs = _decode(lambda a, b: rosa.bf16_input(hq[:, a:b].contiguous(), M),
                      lambda a, b: rosa.bf16_input(hk[:, a:b].contiguous(), M),
                      S, T, K, T0, rle, M)
    q = oracle.discretize_bf16(Hq, M)
    k = oracle.discretize_bf16(Hk, M)
    _check(got, rs, oracle.match_qk(q, k, K, M, rle, cf=True), T0,
           f"qk decode bf16 rle={rle}")


def test_qk_decode_errors():
    """Capacity, the two handle kinds, a run_start output on a step, tables
    without query bits, and the sticky flag for a symbol >= K."""
    S, K, T = 3, 16, 8
    rng = np.random.default_rng(5)
    q = torch.from_numpy(rng.integers(0, K, (S, T)).astype(np.uint8)).to(DEV)
    k = torch.from_numpy(rng.integers(0, K, (S, T)).astype(np.uint8)).to(DEV)
    buf = torch.empty(rosa.rosa_qk_state_bytes(S, K, 4), dtype=torch.uint8, device=DEV)
    h = rosa.rosa_build_qk(rosa.symbols_input(q[:, :2], K),
                           rosa.symbols_input(k[:, :2], K), 0, 4, buf)
    tau = torch.empty(S, dtype=torch.int32, device=DEV)
    for t in (2, 3):
        rosa.rosa_step_qk(h, rosa.symbols_input(q[:, t:t + 1], K),
                          rosa.symbols_input(k[:, t:t + 1], K), rosa.make_qk_out(tau))
    with pytest.raises(rosa.RosaError) as ei:
        rosa.rosa_step_qk(h, rosa.symbols_input(q[:, 4:5], K),
                          rosa.symbols_input(k[:, 4:5], K), rosa.make_qk_out(tau))
    assert ei.value.status == rosa.ROSA_ERR_CAPACITY
    # a self-match step on a query/key handle, and the other way round
    with pytest.raises(rosa.RosaError) as ei:
        rosa.rosa_step(h, rosa.symbols_input(q[:, 4:5], K), None, tau)
    assert ei.value.status == rosa.ROSA_ERR_ARG
    sbuf = torch.empty(rosa.rosa_state_bytes(S, K, 4), dtype=torch.uint8, device=DEV)
    hs = rosa.rosa_build(rosa.symbols_input(q[:, :2], K), 4, sbuf)
    with pytest.raises(rosa.RosaError) as ei:
        rosa.rosa_step_qk(hs, rosa.symbols_input(q[:, 2:3], K),
                          rosa.symbols_input(k[:, 2:3], K), rosa.make_qk_out(tau))
    assert ei.value.status == rosa.ROSA_ERR_ARG
    rosa.rosa_free(hs)
    rosa.rosa_free(h)
    # run_start on a step; tables for an alphabet without query bits
    buf2 = torch.empty(rosa.rosa_qk_state_bytes(S, 3, 8), dtype=torch.uint8, device=DEV)
    q3 = q % 3
    h3 = rosa.rosa_build_qk(rosa.symbols_input(q3[:, :0], 3),
                            rosa.symbols_input(q3[:, :0], 3), 0, 8, buf2)
    with pytest.raises(rosa.RosaError):
        rosa.rosa_step_qk(h3, rosa.symbols_input(q3[:, :1], 3),
                          rosa.symbols_input(q3[:, :1], 3),
                          rosa.make_qk_out(tau, run_start=tau))
    cft = torch.empty((S, 1, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(rosa.RosaError):
        rosa.rosa_step_qk(h3, rosa.symbols_input(q3[:, :1], 3),
                          rosa.symbols_input(q3[:, :1], 3),
                          rosa.make_qk_out(tau, cf_tau=cft))
    # a symbol >= K raises the handle's flag; the step still runs
    bad = torch.full((S, 1), 7, dtype=torch.uint8, device=DEV)
    rosa.rosa_step_qk(h3, rosa.symbols_input(bad, 3), rosa.symbols_input(q3[:, :1], 3),
                      rosa.make_qk_out(tau))
    assert rosa.rosa_state_status(h3) == rosa.ROSA_ERR_SYMBOL
    rosa.rosa_free(h3)


@pytest.mark.parametrize("rle", [False, True])
def test_qk_decode_build_paths(rle):
    """The build's two paths: prefixes of two steps or more and alphabets of
    at most 60 symbols take the batch retrieval plus whole-wave appends, the
    rest walk the prefix in time order.  Edges: a prefix of nearly the whole
    stream, the shortest such prefix, alphabets of 60 and 61 symbols, a
    prefix of exactly two key runs, and a prefix that is a single run."""
    S, T = 4, 480
    for K, T0 in ((16, 470), (16, 2), (60, 300), (61, 300)):
        q, k = _streams(900 + K + T0, S, T, K, "mixed")
        _symbols_case(q, k, K, T0, rle, f"qk decode build K={K} T0={T0} rle={rle}")
    K = 16
    rng = np.random.default_rng(31)
    q = rng.integers(0, K, (S, T)).astype(np.uint8)
    k = rng.integers(0, K, (S, T)).astype(np.uint8)
    k[0, :200] = 3
    k[0, 200:260] = 5                      # two runs, the prefix ends in the second
    k[1, :300] = 7                         # the prefix is one run
    q[2] = k[2]                            # equal streams
    k[3, 250:450] = k[3, 50:250]           # a long repeat across the prefix's end
    q[3, 250:450] = k[3, 250:450]
    _symbols_case(q, k, K, 240, rle, f"qk decode build runs rle={rle}")
