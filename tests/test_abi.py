"""C-ABI checks that need no GPU: the library loads, exports every function
include/rosa.h declares, sizes its buffers, and rejects bad arguments on the
host before anything is launched (no compute call is made here)."""
import ctypes
import os
import re

import pytest

from online_suffix_automaton_amd import rosa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "rosa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rosa_[a-z_]+)\s*\(", src)))


def test_library_exports_header_symbols():
    lib = rosa.load_library()
    names = _declared()
    assert "rosa_match" in names and "rosa_step" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(rosa._SYMBOLS)


def test_error_strings():
    for st in range(7):
        assert rosa.rosa_error_string(st)
    assert "unknown" in rosa.rosa_error_string(99)


def test_workspace_and_state_sizes():
    assert rosa.rosa_match_workspace_bytes(0, 10, 2) == 0
    assert rosa.rosa_match_workspace_bytes(1, 10, 0) == 0
    assert rosa.rosa_match_workspace_bytes(1, 10, 257) == 0
    assert rosa.rosa_match_workspace_bytes(1, 1 << 26, 2) == 0
    a = rosa.rosa_match_workspace_bytes(512, 65536, 16)
    b = rosa.rosa_match_workspace_bytes(512, 65537, 16)
    assert 0 < rosa.rosa_match_workspace_bytes(512, 60000, 16) < a
    # up to 65536 positions the workspace also holds the result records and
    # the deferred answers (16 B per position); beyond, neither
    assert 0 < b and a >= 512 * 65536 * (4 + 16)
    assert rosa.rosa_state_bytes(4, 2, 0) == 0
    s1 = rosa.rosa_state_bytes(512, 16, 66560)
    # dense rows: (2*Tcap-1) states x (16 B node + 4K B row) per stream
    assert s1 >= 512 * (2 * 66560 - 1) * (16 + 64)
    assert rosa.rosa_state_bytes(1, 16, 1) > 0


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _inp(**kw):
    i = rosa.rosa_input()
    i.kind, i.K, i.S, i.T, i.ld = 0, 16, 4, 100, 100
    i.data = FAKE.value
    for k, v in kw.items():
        setattr(i, k, v)
    return i


@pytest.mark.parametrize("bad", [
    dict(kind=7), dict(K=0), dict(K=300), dict(S=0), dict(T=-1),
    dict(T=1 << 26, ld=1 << 26), dict(ld=50), dict(data=None),
    dict(kind=1, M=0, B=1, D=8), dict(kind=1, M=9, B=1, D=9),
    dict(kind=1, M=3, B=1, D=8, ld=8), dict(kind=1, M=4, B=1, D=8, ld=4),
])
def test_match_rejects_bad_input(bad):
    lib = rosa.load_library()
    inp = _inp(**bad)
    out = rosa.rosa_out()
    out.end = FAKE.value
    st = lib.rosa_match(ctypes.byref(inp), ctypes.byref(out), 0x100000, 1 << 30,
                        None)
    assert st == rosa.ROSA_ERR_ARG


def test_match_rejects_bad_buffers():
    lib = rosa.load_library()
    inp = _inp()
    out = rosa.rosa_out()
    out.end = FAKE.value
    # null / misaligned workspace, missing end, too small workspace
    assert lib.rosa_match(ctypes.byref(inp), ctypes.byref(out), None, 1 << 30,
                          None) == rosa.ROSA_ERR_ARG
    assert lib.rosa_match(ctypes.byref(inp), ctypes.byref(out), 0x100010,
                          1 << 30, None) == rosa.ROSA_ERR_ARG
    assert lib.rosa_match(ctypes.byref(inp), None, 0x100000, 1 << 30,
                          None) == rosa.ROSA_ERR_ARG
    out2 = rosa.rosa_out()
    assert lib.rosa_match(ctypes.byref(inp), ctypes.byref(out2), 0x100000,
                          1 << 30, None) == rosa.ROSA_ERR_ARG
    assert lib.rosa_match(ctypes.byref(inp), ctypes.byref(out), 0x100000, 16,
                          None) == rosa.ROSA_ERR_CAPACITY


def test_gather_rejects_bad_arguments():
    lib = rosa.load_library()
    f = lib.rosa_gather
    P = FAKE.value
    assert f(P, 0, 10, 8, 8, 4, P, P, 8, None) == rosa.ROSA_ERR_ARG   # B
    assert f(P, 1, 10, 8, 8, 3, P, P, 8, None) == rosa.ROSA_ERR_ARG   # D % M
    assert f(P, 1, 10, 8, 4, 4, P, P, 8, None) == rosa.ROSA_ERR_ARG   # ldv
    assert f(P, 1, 10, 8, 8, 4, P, P, 4, None) == rosa.ROSA_ERR_ARG   # ldo
    assert f(None, 1, 10, 8, 8, 4, P, P, 8, None) == rosa.ROSA_ERR_ARG
    assert f(P, 1, 10, 8, 8, 9, P, P, 8, None) == rosa.ROSA_ERR_ARG   # M


def test_state_api_rejects_bad_handles_and_args():
    lib = rosa.load_library()
    assert lib.rosa_state_length(None) == -1
    assert lib.rosa_state_status(None, None) == rosa.ROSA_ERR_STATE
    lib.rosa_free(None)   # ignored
    inp = _inp(T=1, ld=1)
    end = FAKE.value
    assert lib.rosa_step(None, ctypes.byref(inp), None, 0, 0, end, None, None,
                         0, None) == rosa.ROSA_ERR_STATE
    h = ctypes.c_void_p()
    # capacity below T, misaligned or null buffer, too small buffer
    inp2 = _inp()
    assert lib.rosa_build(ctypes.byref(inp2), 50, 0x100000, 1 << 30,
                          ctypes.byref(h), None, None) == rosa.ROSA_ERR_ARG
    assert lib.rosa_build(ctypes.byref(inp2), 200, 0x100010, 1 << 30,
                          ctypes.byref(h), None, None) == rosa.ROSA_ERR_ARG
    assert lib.rosa_build(ctypes.byref(inp2), 200, None, 1 << 30,
                          ctypes.byref(h), None, None) == rosa.ROSA_ERR_ARG
    assert lib.rosa_build(ctypes.byref(inp2), 200, 0x100000, 64,
                          ctypes.byref(h), None, None) == rosa.ROSA_ERR_CAPACITY
    assert not h.value


def test_state_api_never_reads_unknown_handles():
    """Handles are looked up in the library's registry of live handles
    before they are read: a pointer the library never returned (here one
    into unmapped memory, which would fault if read) is rejected, and a
    double free is ignored."""
    lib = rosa.load_library()
    bogus = ctypes.c_void_p(0x10)
    assert lib.rosa_state_length(bogus) == -1
    assert lib.rosa_state_status(bogus, None) == rosa.ROSA_ERR_STATE
    inp = _inp(T=1, ld=1)
    assert lib.rosa_step(bogus, ctypes.byref(inp), None, 0, 0, FAKE.value,
                         None, None, 0, None) == rosa.ROSA_ERR_STATE
    lib.rosa_free(bogus)
    lib.rosa_free(bogus)


def test_gather_and_scatter_bindings_check_layouts():
    """The binding refuses tensors whose layout the C-ABI would read wrongly
    (CPU tensors never reach the library: the device check comes first, so
    the layout checks are exercised through the helpers)."""
    import torch
    V = torch.zeros((2, 10, 8), dtype=torch.int16)
    rosa._rows_3d(V, "V")
    with pytest.raises(ValueError):
        rosa._rows_3d(torch.zeros((2, 20, 8), dtype=torch.int16)[:, :10], "V")
    with pytest.raises(ValueError):
        rosa._rows_3d(V, "out", (2, 10, 4))
    with pytest.raises(ValueError):
        rosa._rows_3d(torch.zeros((2, 8, 10), dtype=torch.int16).transpose(1, 2), "V")
    rosa._end_rows(torch.zeros((4, 10), dtype=torch.int32), 4, 10)
    with pytest.raises(ValueError):
        rosa._end_rows(torch.zeros((4, 10), dtype=torch.int64), 4, 10)
    with pytest.raises(ValueError):
        rosa._end_rows(torch.zeros((4, 11), dtype=torch.int32), 4, 10)


def test_match_qk_rejects_bad_arguments():
    lib = rosa.load_library()
    f = lib.rosa_match_qk
    assert rosa.rosa_match_qk_workspace_bytes(0, 10, 2) == 0
    assert rosa.rosa_match_qk_workspace_bytes(4, 100, 16) > 0
    q, k = _inp(), _inp()
    out = rosa.rosa_qk_out()
    out.tau = FAKE.value
    big = 1 << 40
    ws = 0x100000

    def call(q_, k_, flags=0, o=out, w=ws, nb=big):
        return f(ctypes.byref(q_), ctypes.byref(k_), flags,
                 ctypes.byref(o) if o is not None else None, w, nb, None)
    assert call(q, _inp(T=99)) == rosa.ROSA_ERR_ARG          # T differs
    assert call(q, _inp(S=3)) == rosa.ROSA_ERR_ARG           # S differs
    assert call(q, _inp(K=8)) == rosa.ROSA_ERR_ARG           # K differs
    assert call(q, k, flags=2) == rosa.ROSA_ERR_ARG          # unknown flag
    assert call(q, k, o=None) == rosa.ROSA_ERR_ARG
    assert call(q, k, o=rosa.rosa_qk_out()) == rosa.ROSA_ERR_ARG   # no tau
    assert call(q, k, w=0x100010) == rosa.ROSA_ERR_ARG       # misaligned
    assert call(q, k, nb=64) == rosa.ROSA_ERR_CAPACITY
    # counterfactual tables need K = 2^M
    o2 = rosa.rosa_qk_out()
    o2.tau, o2.cf_tau = FAKE.value, FAKE.value
    assert call(_inp(K=3), _inp(K=3), o=o2) == rosa.ROSA_ERR_ARG
    assert call(_inp(K=1), _inp(K=1), o=o2) == rosa.ROSA_ERR_ARG


def test_scatter_grad_rejects_bad_arguments():
    lib = rosa.load_library()
    f = lib.rosa_scatter_grad
    P = FAKE.value
    assert rosa.rosa_scatter_grad_workspace_bytes(0, 10) == 0
    assert rosa.rosa_scatter_grad_workspace_bytes(4, 10) > 0
    ws, big = 0x100000, 1 << 40
    assert f(P, 0, 10, 8, 8, 4, P, P, 8, ws, big, None) == rosa.ROSA_ERR_ARG  # B
    assert f(P, 1, 10, 8, 8, 3, P, P, 8, ws, big, None) == rosa.ROSA_ERR_ARG  # D % M
    assert f(P, 1, 10, 8, 8, 9, P, P, 8, ws, big, None) == rosa.ROSA_ERR_ARG  # M
    assert f(P, 1, 10, 8, 4, 4, P, P, 8, ws, big, None) == rosa.ROSA_ERR_ARG  # ldt
    assert f(P, 1, 10, 8, 8, 4, P, P, 4, ws, big, None) == rosa.ROSA_ERR_ARG  # ldg
    assert f(None, 1, 10, 8, 8, 4, P, P, 8, ws, big, None) == rosa.ROSA_ERR_ARG
    assert f(P, 1, 10, 8, 8, 4, P, P, 8, 0x100010, big, None) == rosa.ROSA_ERR_ARG
    assert f(P, 1, 10, 8, 8, 4, P, P, 8, ws, 16, None) == rosa.ROSA_ERR_CAPACITY


def test_qk_decode_api_rejects_bad_handles_and_args():
    """The query/key decode entry points validate on the host: sizes,
    unknown handles, mismatched inputs, flags, capacity below the prefix,
    misaligned or short buffers, tables for an alphabet without query bits.
    Nothing here reaches a kernel."""
    lib = rosa.load_library()
    assert lib.rosa_qk_state_bytes(0, 16, 10) == 0
    assert lib.rosa_qk_state_bytes(4, 0, 10) == 0
    assert lib.rosa_qk_state_bytes(4, 257, 10) == 0
    assert lib.rosa_qk_state_bytes(4, 16, 0) == 0
    assert lib.rosa_qk_state_bytes(4, 16, 1 << 26) == 0
    # per stream: (2*Tcap-1) records of 16 + 4K bytes and a start time per step
    assert lib.rosa_qk_state_bytes(8, 16, 1000) >= 8 * (1999 * 128 + 4 * 1000)
    row = _inp(T=1, ld=1)
    out = rosa.rosa_qk_out()
    out.tau = FAKE.value
    for h in (None, ctypes.c_void_p(0x10)):
        assert lib.rosa_step_qk(h, ctypes.byref(row), ctypes.byref(row),
                                ctypes.byref(out), None) == rosa.ROSA_ERR_STATE
    h = ctypes.c_void_p()
    q, k = _inp(), _inp()
    ok_buf, big = 0x100000, 1 << 40

    def build(qq=q, kk=k, flags=0, cap=200, buf=ok_buf, nb=big, o=None):
        return lib.rosa_build_qk(ctypes.byref(qq), ctypes.byref(kk), flags, cap,
                                 buf, nb, ctypes.byref(h),
                                 ctypes.byref(o) if o is not None else None, None)
    assert build(kk=_inp(T=99)) == rosa.ROSA_ERR_ARG          # shapes differ
    assert build(kk=_inp(K=8)) == rosa.ROSA_ERR_ARG
    assert build(flags=2) == rosa.ROSA_ERR_ARG                 # unknown flag
    assert build(cap=50) == rosa.ROSA_ERR_ARG                  # capacity < T
    assert build(buf=0x100010) == rosa.ROSA_ERR_ARG            # not 256-aligned
    assert build(buf=None) == rosa.ROSA_ERR_ARG
    assert build(nb=64) == rosa.ROSA_ERR_CAPACITY
    noto = rosa.rosa_qk_out()                                   # tau missing
    assert build(o=noto) == rosa.ROSA_ERR_ARG
    cf = rosa.rosa_qk_out()
    cf.tau, cf.cf_tau = FAKE.value, FAKE.value
    assert build(qq=_inp(K=3), kk=_inp(K=3), o=cf) == rosa.ROSA_ERR_ARG
    assert not h.value


def test_discretize_rejects_bad_arguments():
    lib = rosa.load_library()
    sym = _inp()                                   # a symbols input
    assert lib.rosa_discretize(ctypes.byref(sym), FAKE.value, 100, None) == rosa.ROSA_ERR_ARG
    bf = _inp(kind=1, M=4, B=1, D=8, ld=8, T=100)
    assert lib.rosa_discretize(ctypes.byref(bf), None, 100, None) == rosa.ROSA_ERR_ARG
    assert lib.rosa_discretize(ctypes.byref(bf), FAKE.value, 99, None) == rosa.ROSA_ERR_ARG
    empty = _inp(kind=1, M=4, B=1, D=8, ld=8, T=0)
    assert lib.rosa_discretize(ctypes.byref(empty), None, 0, None) == rosa.ROSA_OK
