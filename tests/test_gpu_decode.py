"""GPU parity of the online path: rosa_build over a prefix followed by
rosa_step per new position must give, at every position, the outputs the
oracle computes over the whole stream (online == offline), plus the gathered
value row."""
import numpy as np
import pytest
import torch

import oracle
from online_suffix_automaton_amd import rosa, synth

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _dev(a):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _state(S, K, cap):
    nb = rosa.rosa_state_bytes(S, K, cap)
    return torch.empty(nb, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("K,T0,n", [(2, 0, 40), (4, 1, 60), (16, 300, 120),
                                    (256, 77, 30), (1, 50, 20)])
def test_symbols_build_then_steps(K, T0, n):
    rng = np.random.default_rng(K * 100 + T0)
    S = 7
    full = rng.integers(0, K, size=(S, T0 + n), dtype=np.uint8)
    Eo, SYMo, Lo = oracle.match(full, K)
    cap = T0 + n
    buf = _state(S, K, cap)
    E0 = torch.empty((S, max(T0, 1)), dtype=torch.int32, device=DEV)
    S0 = torch.empty((S, max(T0, 1)), dtype=torch.int16, device=DEV)
    L0 = torch.empty((S, max(T0, 1)), dtype=torch.int32, device=DEV)
    pre = _dev(full[:, :T0]) if T0 > 0 else torch.empty((S, 0), dtype=torch.uint8,
                                                         device=DEV)
    st = rosa.rosa_build(rosa.symbols_input(pre, K), cap, buf,
                         rosa.make_out(E0, S0, L0))
    if T0 > 0:
        assert np.array_equal(E0.cpu().numpy(), Eo[:, :T0])
        assert np.array_equal(S0.cpu().numpy(), SYMo[:, :T0])
        assert np.array_equal(L0.cpu().numpy(), Lo[:, :T0])
    rows = _dev(full)
    end = torch.empty(S, dtype=torch.int32, device=DEV)
    sym = torch.empty(S, dtype=torch.int16, device=DEV)
    for t in range(T0, T0 + n):
        r = rows[:, t:t + 1]
        rosa.rosa_step(st, rosa.symbols_input(r, K), None, end, sym)
        e, s_ = end.cpu().numpy(), sym.cpu().numpy()
        assert np.array_equal(e, Eo[:, t]), f"t={t}"
        assert np.array_equal(s_, SYMo[:, t]), f"t={t}"
    assert rosa.rosa_state_length(st) == T0 + n
    with pytest.raises(rosa.RosaError) as ei:
        rosa.rosa_step(st, rosa.symbols_input(rows[:, :1], K), None, end, sym)
    assert ei.value.status == rosa.ROSA_ERR_CAPACITY
    assert rosa.rosa_state_status(st) == rosa.ROSA_OK


def test_bf16_build_steps_with_gather():
    B, D, M, T0, n = 2, 32, 4, 500, 64
    Tc = T0 + n
    H = synth.bf16_normal((B, Tc, D), 31)
    V = synth.bf16_normal((B, Tc, D), 32)
    so = oracle.discretize_bf16(H, M)
    Eo, SYMo, Lo = oracle.match(so, 16)
    go = oracle.gather(V, Eo, M)
    S = B * D // M
    buf = _state(S, 16, Tc)
    Hd, Vd = _dev(H), _dev(V)
    st = rosa.rosa_build(rosa.bf16_input(Hd[:, :T0].contiguous(), M), Tc, buf)
    end = torch.empty(S, dtype=torch.int32, device=DEV)
    sym = torch.empty(S, dtype=torch.int16, device=DEV)
    orow = torch.empty((B, D), dtype=torch.int16, device=DEV)
    for t in range(T0, Tc):
        row = Hd[:, t:t + 1].contiguous()
        rosa.rosa_step(st, rosa.bf16_input(row, M), Vd, end, sym, orow)
        assert np.array_equal(end.cpu().numpy(), Eo[:, t]), f"t={t}"
        assert np.array_equal(sym.cpu().numpy(), SYMo[:, t]), f"t={t}"
        assert np.array_equal(orow.cpu().numpy().view(np.uint16), go[:, t]), f"t={t}"


def test_step_symbol_flag():
    K, S = 4, 3
    buf = _state(S, K, 10)
    x = _dev(np.zeros((S, 2), dtype=np.uint8))
    st = rosa.rosa_build(rosa.symbols_input(x, K), 10, buf)
    end = torch.empty(S, dtype=torch.int32, device=DEV)
    bad = _dev(np.array([[1], [7], [2]], dtype=np.uint8))
    rosa.rosa_step(st, rosa.symbols_input(bad, K), None, end)
    assert rosa.rosa_state_status(st) == rosa.ROSA_ERR_SYMBOL


def test_decode_workload():
    """The decode workload: 512 streams, 65,536-position prefix from the long
    workload's generator, then 1024 appended positions, one step each."""
    _say("generating")
    pre = synth.long()
    tail = synth.decode_tail()
    H = np.concatenate([pre["H"], tail["H"]], axis=1)
    V = np.concatenate([pre["V"], tail["V"]], axis=1)
    T0, n = pre["H"].shape[1], tail["H"].shape[1]
    Tc = T0 + n
    S = 512
    buf = _state(S, 16, Tc)
    Hd, Vd = _dev(H), _dev(V)
    _say("build")
    st = rosa.rosa_build(rosa.bf16_input(Hd[:, :T0], 4), Tc, buf)
    torch.cuda.synchronize()
    ends = torch.empty((n, S), dtype=torch.int32, device=DEV)
    syms = torch.empty((n, S), dtype=torch.int16, device=DEV)
    orows = torch.empty((n, 2048), dtype=torch.int16, device=DEV)
    _say("steps")
    for i in range(n):
        row = Hd[:, T0 + i:T0 + i + 1]
        rosa.rosa_step(st, rosa.bf16_input(row, 4), Vd, ends[i], syms[i],
                       orows[i:i + 1])
    torch.cuda.synchronize()
    _say("oracle")
    so = oracle.discretize_bf16(H, 4)
    Eo, SYMo, Lo = oracle.match(so, 16)
    assert np.array_equal(ends.cpu().numpy(), Eo[:, T0:].T)
    assert np.array_equal(syms.cpu().numpy(), SYMo[:, T0:].T)
    go = oracle.gather(V, Eo, 4)[0, T0:]
    assert np.array_equal(orows.cpu().numpy().view(np.uint16), go)


def test_structured_build_then_steps():
    """Streams with long recurrences (periodic, Fibonacci word, planted
    copies, constant): many clones and long suffix paths across the
    build/step boundary and from step to step."""
    T0, n = 700, 150
    T = T0 + n
    rows = [synth.periodic(T, [0, 1]), synth.fibonacci_word(T), synth.constant(T),
            synth.planted_copies(T, 4, 5, gap_mean=30, len_lo=10, len_hi=120),
            synth.periodic(T, [0, 1, 2, 0, 1])]
    full = np.stack([np.asarray(r, dtype=np.uint8) for r in rows])
    S, K = full.shape[0], 4
    Eo, SYMo, Lo = oracle.match(full, K)
    buf = _state(S, K, T)
    E0 = torch.empty((S, T0), dtype=torch.int32, device=DEV)
    st = rosa.rosa_build(rosa.symbols_input(_dev(full[:, :T0]), K), T, buf,
                         rosa.make_out(E0, None, None))
    assert np.array_equal(E0.cpu().numpy(), Eo[:, :T0])
    rows_d = _dev(full)
    end = torch.empty(S, dtype=torch.int32, device=DEV)
    sym = torch.empty(S, dtype=torch.int16, device=DEV)
    for t in range(T0, T):
        rosa.rosa_step(st, rosa.symbols_input(rows_d[:, t:t + 1], K), None, end, sym)
        assert np.array_equal(end.cpu().numpy(), Eo[:, t]), f"t={t}"
        assert np.array_equal(sym.cpu().numpy(), SYMo[:, t]), f"t={t}"
