"""rosa_match_noalloc: rosa_match with its workspace in the library's fixed
device array (for callers that cannot allocate).  Through the C-ABI, its
outputs must equal rosa_match's bit for bit; two calls in a row, the second
on a smaller input, check that nothing left from the first call leaks into
the second.  Shapes beyond the array are rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

from online_suffix_automaton_amd import rosa, synth

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _outs(S, T):
    E = torch.full((S, T), -7, dtype=torch.int32, device=DEV)
    SYM = torch.full((S, T), -7, dtype=torch.int16, device=DEV)
    L = torch.full((S, T), -7, dtype=torch.int32, device=DEV)
    syms = torch.full((S, T), 0xEE, dtype=torch.uint8, device=DEV)
    return (E, SYM, L, syms), rosa.make_out(E, SYM, L, syms)


def _both(inp, S, T, K):
    """Outputs of rosa_match (own workspace) and rosa_match_noalloc."""
    a, oa = _outs(S, T)
    b, ob = _outs(S, T)
    ws = torch.empty(rosa.rosa_match_workspace_bytes(S, T, K), dtype=torch.uint8,
                     device=DEV)
    rosa.rosa_match(inp, oa, ws)
    rosa.rosa_match_noalloc(inp, ob)
    torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    for name, x, y in zip(("E", "SYM", "L", "symbols"), a, b):
        if not torch.equal(x, y):
            bad = torch.nonzero(x != y)
            raise AssertionError(f"{what}: {name} differs at {len(bad)} places, "
                                 f"first {bad[0].tolist()}")


@pytest.mark.gpu
def test_noalloc_equals_match_twice_second_smaller():
    # first call: the batched shape, bf16 [8, 4096, 256], M = 4 -> 512 x 4096
    B, T, D, M = 8, 4096, 256, 4
    _say(f"noalloc call 1: bf16 [{B},{T},{D}] M={M}")
    H = synth.bf16_normal((B, T, D), 2)
    Hd = torch.from_numpy(H.view(np.int16)).to(DEV)
    S = B * D // M
    assert rosa.rosa_match_workspace_bytes(S, T, 16) <= \
        rosa.ROSA_NOALLOC_MAX_WORKSPACE_BYTES
    a, b = _both(rosa.bf16_input(Hd, M), S, T, 16)
    _same(a, b, "call 1")
    # second call: fewer, shorter streams with structure (long repeats take
    # the deferred-answer path), symbols input
    S2, T2, K2 = 5, 3001, 16
    _say(f"noalloc call 2: symbols [{S2},{T2}] K={K2}")
    rng = np.random.default_rng(5)
    x = rng.integers(0, K2, (S2, T2)).astype(np.uint8)
    x[1, 1500:2500] = x[1, 100:1100]
    x[2, :] = 3
    x[3, 1::2] = x[3, 0:-1:2]
    xd = torch.from_numpy(x).to(DEV)
    a2, b2 = _both(rosa.symbols_input(xd, K2), S2, T2, K2)
    _same(a2, b2, "call 2")
    # a third, tiny binary call after the other two
    S3, T3 = 3, 257
    x3 = rng.integers(0, 2, (S3, T3)).astype(np.uint8)
    a3, b3 = _both(rosa.symbols_input(torch.from_numpy(x3).to(DEV), 2), S3, T3, 2)
    _same(a3, b3, "call 3")


def test_noalloc_rejects_on_host():
    """Checked before any device work: shapes beyond the array and bad
    arguments (no GPU needed)."""
    lib = rosa.load_library()
    fake = 0x1000   # never dereferenced: validation fails first
    inp = rosa.rosa_input()
    inp.kind, inp.K, inp.S, inp.T, inp.ld = rosa.ROSA_IN_SYMBOLS, 16, 512, 65536, 65536
    inp.data = fake
    out = rosa.rosa_out()
    out.end = fake
    assert rosa.rosa_match_workspace_bytes(512, 65536, 16) > \
        rosa.ROSA_NOALLOC_MAX_WORKSPACE_BYTES
    st = lib.rosa_match_noalloc(ctypes.byref(inp), ctypes.byref(out), None)
    assert st == rosa.ROSA_ERR_CAPACITY
    inp.K = 0
    assert lib.rosa_match_noalloc(ctypes.byref(inp), ctypes.byref(out), None) \
        == rosa.ROSA_ERR_ARG
    inp.K = 16
    out.end = None
    assert lib.rosa_match_noalloc(ctypes.byref(inp), ctypes.byref(out), None) \
        == rosa.ROSA_ERR_ARG
