"""GPU parity: the HIP path through the C-ABI against the CPU oracle.

Every integer output (E, SYM, L, packed symbols) must be bit-exact, and the
gathered bf16 values byte-identical.  Cases span several tiles and ragged
tails, every alphabet size class, structured streams that defeat the bucket
fast path, and the full-size workloads.
"""
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


def _check(E, SYM, L, Eo, SYMo, Lo, what):
    E, SYM, L = E.cpu().numpy(), SYM.cpu().numpy(), L.cpu().numpy()
    for name, a, b in (("E", E, Eo), ("SYM", SYM, SYMo), ("L", L, Lo)):
        if not np.array_equal(a, b):
            bad = np.argwhere(a != b)
            s, t = bad[0]
            raise AssertionError(
                f"{what}: {name} differs at {len(bad)} places, first (s={s}, "
                f"t={t}): gpu {a[s, t]} oracle {b[s, t]}")


def _run_symbols(sym, K, what):
    """Symbol rows through rosa_match, checked against the oracle twice:
    contiguous rows with the packed-symbol copy requested (the rows are first
    copied into the workspace), and the same rows at a pitch of a multiple of
    16 bytes (streams of at most 65536 positions: the retrieval kernel reads
    them itself).  The bytes past T in the second hold 255, a symbol >= K for
    every K < 256, so a read of them would raise the symbol flag."""
    x = _dev(sym)
    E, SYM, L, syms = rosa.match(x, K=K, want_symbols=True)
    torch.cuda.synchronize()
    Eo, SYMo, Lo = oracle.match(sym, K)
    _check(E, SYM, L, Eo, SYMo, Lo, what)
    assert np.array_equal(syms.cpu().numpy(), sym)
    S, T = sym.shape
    if S > 1 and T <= 65536:
        ld = (T + 15) // 16 * 16 + 16
        buf = torch.full((S, ld), 255, dtype=torch.uint8, device=DEV)
        buf[:, :T] = x
        ws = torch.empty(rosa.rosa_match_workspace_bytes(S, T, K), dtype=torch.uint8,
                         device=DEV)
        E2, SYM2, L2, _ = rosa.match(buf[:, :T], K=K, ws=ws)
        assert rosa.rosa_match_status(ws) == rosa.ROSA_OK, what + " (aligned rows)"
        _check(E2, SYM2, L2, Eo, SYMo, Lo, what + " (aligned rows)")
    return E


def test_tiny_workload():
    w = synth.tiny()
    _run_symbols(w["sym"], w["K"], "tiny")


@pytest.mark.parametrize("K", [1, 2, 3, 4, 16, 17, 256])
def test_random_streams_all_alphabets(K):
    rng = np.random.default_rng(100 + K)
    for T in (1, 2, 3, 5, 17, 64, 65, 100, 257, 1000, 4099):
        S = int(rng.integers(1, 9))
        sym = rng.integers(0, K, size=(S, T), dtype=np.uint8)
        _say(f"K={K} S={S} T={T}")
        _run_symbols(sym, K, f"random K={K} T={T}")


@pytest.mark.parametrize("T", [8192, 65536])
def test_last_new_dgram_late(T):
    """The positions with L < d end at the latest first occurrence of a
    d-gram; the short-match scan stops there and spreads its segments over
    that range.  Streams whose last new d-gram sits at chosen places: the
    very end, chunk and segment boundaries, mid-stream, early (a periodic
    stream), after a random prefix."""
    rng = np.random.default_rng(7 + T)
    K = 16
    base = np.resize(np.array([0, 1, 2, 3, 4, 5, 6], dtype=np.uint8), T)
    rows = []
    for q in (T - 1, T - 2, T - 3, T // 2, T // 16 * 3 - 1, T // 16 * 3,
              4095, 4096, 63, 64):
        r = base.copy()
        r[q] = 15   # new d-grams end at q .. q+d-1 (inside the stream)
        rows.append(r)
    rows.append(base.copy())
    for pre in (100, T // 3, T - 70):
        r = base.copy()
        r[:pre] = rng.integers(0, K, pre)
        rows.append(r)
    sym = np.stack(rows)
    _say(f"late new d-grams: S={sym.shape[0]} T={T}")
    _run_symbols(sym, K, f"late new d-grams T={T}")


def test_structured_streams():
    T = 3000
    rows = [synth.constant(T), synth.periodic(T, [0, 1]),
            synth.periodic(T, [0, 1, 2]), synth.periodic(T, [0, 0, 1]),
            synth.fibonacci_word(T), np.resize(synth.de_bruijn(2, 10), T),
            synth.planted_copies(T, 4, 11, gap_mean=40, len_lo=20, len_hi=200),
            synth.planted_copies(T, 16, 12, gap_mean=100, len_lo=32, len_hi=512)]
    sym = np.stack([r.astype(np.uint8) for r in rows])
    for K in (16, 256):
        _say(f"structured K={K}")
        _run_symbols(sym, K, f"structured K={K}")


def test_constant_and_periodic_long():
    # one bucket holds (nearly) the whole stream: large-group path only
    T = 8192
    sym = np.stack([synth.constant(T, 1), synth.periodic(T, [2, 5]),
                    synth.periodic(T, [0, 1, 2, 3, 4, 5, 6])])
    _run_symbols(sym, 8, "constant/periodic 8192")


def _closed_form_periodic(T, p):
    """E, L of a stream of period p with p distinct symbols (the oracle's
    closed form, pinned in tests/test_oracle.py): no match before t = p,
    then the suffix of length t-p+1 ends at t-p; p = 1 is the constant
    stream."""
    t = np.arange(T)
    E = np.where(t < p, -1, t - p).astype(np.int32)
    L = np.where(t < p, 0, t - p + 1).astype(np.int32)
    return E, L


def test_low_entropy_streams_at_65536():
    """Constant and periodic streams of 65,536 positions: one bucket holds
    (nearly) the whole stream and stays uniform level after level; the
    large-bucket solver defers such groups to the time-ordered pass (the
    extension rule), so the call is O(T) per stream instead of O(T^2).
    Checked against the closed forms; streams mixing constant stretches with
    random ones against the oracle."""
    T = 65536
    rows, forms = [], []
    for sym0, p in ((5, 1), (0, 1), (None, 3), (None, 7), (None, 2)):
        x = synth.constant(T, sym0) if p == 1 else synth.periodic(T, list(range(p)))
        rows.append(np.asarray(x, dtype=np.uint8))
        forms.append(_closed_form_periodic(T, p))
    x = np.stack(rows)
    xd = _dev(x)
    E, SYM, L, _ = rosa.match(xd, K=16)
    torch.cuda.synchronize()
    E, L, SYM = E.cpu().numpy(), L.cpu().numpy(), SYM.cpu().numpy()
    for i, (Ef, Lf) in enumerate(forms):
        assert np.array_equal(E[i], Ef), f"low-entropy stream {i}: E"
        assert np.array_equal(L[i], Lf), f"low-entropy stream {i}: L"
        want_sym = np.where(Ef >= 0, x[i][np.maximum(Ef, -1) + 1].astype(np.int16), -1)
        assert np.array_equal(SYM[i], want_sym), f"low-entropy stream {i}: SYM"
    # constant stretches inside random streams (the oracle's cost grows
    # with the square of a constant stretch, so these stay moderate)
    rng = np.random.default_rng(31)
    mixed = []
    for lo, hi in ((1000, 21000), (40000, 60000), (0, 15000)):
        m = rng.integers(0, 16, T).astype(np.uint8)
        m[lo:hi] = 9
        mixed.append(m)
    m = rng.integers(0, 16, T).astype(np.uint8)
    m[5000:25000] = np.tile(np.array([1, 4, 1, 6], np.uint8), 5000)
    mixed.append(m)
    _say("mixed constant/periodic stretches T=65536")
    _run_symbols(np.stack(mixed), 16, "low-entropy stretches 65536")


def test_mixed_bucket_sizes():
    # some streams random, some low-entropy, in one call
    rng = np.random.default_rng(7)
    T = 20000
    rows = [rng.integers(0, 16, T), rng.integers(0, 2, T),
            synth.periodic(T, list(range(16))), rng.integers(0, 3, T) * 5,
            synth.planted_copies(T, 16, 3)]
    sym = np.stack([np.asarray(r, dtype=np.uint8) for r in rows])
    _run_symbols(sym, 16, "mixed")


def test_lds_path_maximum_length():
    """T = 65536, the longest stream the LDS-resident kernel takes, with a
    small alphabet (deep bucketing, d = 11 for K = 2) and K = 16."""
    rng = np.random.default_rng(21)
    T = 65536
    for K in (2, 16):
        sym = rng.integers(0, K, size=(2, T), dtype=np.uint8)
        _say(f"T={T} K={K}")
        _run_symbols(sym, K, f"T={T} K={K}")


def test_streams_longer_than_lds_path():
    """T > 65536 takes the kernel with symbols and buckets in HBM: random
    streams of two alphabets, planted copies, a periodic stream, and T
    one past the LDS limit."""
    rng = np.random.default_rng(22)
    for T in (65537, 100003):
        rows = [rng.integers(0, 16, T), rng.integers(0, 4, T),
                synth.planted_copies(T, 16, 23), synth.periodic(T, [1, 2, 3, 5, 8])]
        sym = np.stack([np.asarray(r, dtype=np.uint8) for r in rows])
        _say(f"T={T} (HBM path)")
        _run_symbols(sym, 16, f"T={T}")


@pytest.mark.parametrize("K,T,ld", [(16, 1000, 1024), (10, 1000, 1024),
                                    (16, 65536, 65536), (10, 50001, 50016)])
def test_symbol_out_of_range_flag_wide_rows(K, T, ld):
    """The symbol check where the retrieval kernel reads 16-byte aligned
    caller rows itself (row pitch a multiple of 16 bytes; streams short
    enough for that kernel to run the time-ordered pass too, and streams
    long enough that it writes the padded rows out for the later kernel): a
    symbol >= K in the middle of a row (a whole chunk: a mask test for K a
    power of two, byte compares otherwise) and at its last position (the
    byte path when T is not a multiple of 16) raise the flag; rows without
    one do not, and then give the oracle's outputs."""
    rng = np.random.default_rng(40 + K + T)
    S = 3
    base = rng.integers(0, K, size=(S, ld), dtype=np.uint8)
    x = _dev(base)[:, :T]
    ws = torch.empty(rosa.rosa_match_workspace_bytes(S, T, K), dtype=torch.uint8,
                     device=DEV)
    _say(f"wide rows K={K} T={T} ld={ld}")
    E, SYM, L, _ = rosa.match(x, K=K, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_OK
    Eo, SYMo, Lo = oracle.match(np.ascontiguousarray(base[:, :T]), K)
    _check(E, SYM, L, Eo, SYMo, Lo, f"wide rows K={K} T={T}")
    for where in (517, T - 1):
        bad = base.copy()
        bad[1, where] = K + 3
        rosa.match(_dev(bad)[:, :T], K=K, ws=ws)
        assert rosa.rosa_match_status(ws) == rosa.ROSA_ERR_SYMBOL, where
    # the report belongs to the last call on the workspace, whichever path
    # each call took: these rows are read by the retrieval kernel itself,
    # which stores a status slot per stream and clears nothing first; with
    # the packed-symbol copy requested the rows are copied into the
    # workspace first, by a kernel that reports into the cleared header
    x_bad = _dev(bad)[:, :T]
    rosa.match(x, K=K, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_OK, "good after bad"
    rosa.match(x_bad, K=K, ws=ws, want_symbols=True)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_ERR_SYMBOL, "copy path, bad"
    rosa.match(x, K=K, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_OK, "own rows after copy path"
    rosa.match(x_bad, K=K, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_ERR_SYMBOL, "own rows, bad"
    rosa.match(x, K=K, ws=ws, want_symbols=True)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_OK, "copy path after own rows"
    # fewer streams on the same workspace: only their slots count
    rosa.match(x_bad, K=K, ws=ws)
    rosa.match(x[:1], K=K, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_OK, "one stream after three"


@pytest.mark.parametrize("M,pad", [(4, 0), (4, 37), (3, 5), (8, 0), (1, 16)])
def test_discretize_alone(M, pad):
    """rosa_discretize: the symbols of a bf16 input into caller rows (row
    stride T + pad), equal to the oracle's discretization on every bf16
    pattern class (the hidden states include all 65,536 patterns), and
    rosa_match over those rows equals rosa_match over the bf16 input."""
    B, T, D = 2, 2048, 32 * M
    H = synth.bf16_normal((B, T, D), 90 + M)
    H.reshape(-1)[:65536] = np.arange(65536, dtype=np.uint16)
    S = B * D // M
    Hd = _dev(H.view(np.int16))
    buf = torch.full((S, T + pad), 0xEE, dtype=torch.uint8, device=DEV)
    syms = buf[:, :T]
    rosa.rosa_discretize(rosa.bf16_input(Hd, M), syms)
    want = oracle.discretize_bf16(H, M)
    assert np.array_equal(syms.cpu().numpy(), want)
    if pad:
        assert bool((buf[:, T:] == 0xEE).all()), "bytes past T were written"
    E1, SYM1, L1, _ = rosa.match(Hd, M=M)
    E2, SYM2, L2, _ = rosa.match(syms, K=1 << M)
    assert torch.equal(E1, E2) and torch.equal(SYM1, SYM2) and torch.equal(L1, L2)


def test_strided_symbol_rows():
    rng = np.random.default_rng(8)
    base = rng.integers(0, 16, size=(6, 1500), dtype=np.uint8)
    x = _dev(base)[:, :1333]          # rows with stride 1500 > T
    E, SYM, L, _ = rosa.match(x, K=16)
    Eo, SYMo, Lo = oracle.match(np.ascontiguousarray(base[:, :1333]), 16)
    _check(E, SYM, L, Eo, SYMo, Lo, "strided rows")


def test_symbol_out_of_range_flag():
    sym = np.array([[0, 1, 2, 9, 1]], dtype=np.uint8)
    x = _dev(sym)
    ws = torch.empty(rosa.rosa_match_workspace_bytes(1, 5, 4), dtype=torch.uint8,
                     device=DEV)
    rosa.match(x, K=4, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_ERR_SYMBOL
    x2 = _dev(np.array([[0, 1, 2, 3, 1]], dtype=np.uint8))
    rosa.match(x2, K=4, ws=ws)
    assert rosa.rosa_match_status(ws) == rosa.ROSA_OK


def test_bf16_threshold_all_patterns():
    # one position, 65536 channels, M = 1: symbol = I[h > 0]
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(1, 1, -1)
    E, SYM, L, syms = rosa.match(_dev(bits), M=1, want_symbols=True)
    want = oracle.discretize_bf16(bits, 1)
    assert np.array_equal(syms.cpu().numpy(), want)
    assert (E.cpu().numpy() == -1).all()


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_bf16_small_all_widths(M):
    B, T, D = 3, 333, 24 if M != 8 else 32
    H = synth.bf16_normal((B, T, D), 20 + M)
    E, SYM, L, syms = rosa.match(_dev(H), M=M, want_symbols=True)
    so = oracle.discretize_bf16(H, M)
    assert np.array_equal(syms.cpu().numpy(), so)
    Eo, SYMo, Lo = oracle.match(so, 1 << M)
    _check(E, SYM, L, Eo, SYMo, Lo, f"bf16 M={M}")


def test_batched_workload():
    w = synth.batched()
    H = w["H"]
    E, SYM, L, syms = rosa.match(_dev(H), M=4, want_symbols=True)
    torch.cuda.synchronize()
    so = oracle.discretize_bf16(H, 4)
    assert np.array_equal(syms.cpu().numpy(), so)
    Eo, SYMo, Lo = oracle.match(so, 16)
    _check(E, SYM, L, Eo, SYMo, Lo, "batched")


def test_repeat_workload():
    _say("generating repeat workload")
    w = synth.repeat()
    _say("gpu")
    x = _dev(w["sym"])
    E, SYM, L, _ = rosa.match(x, K=16)
    torch.cuda.synchronize()
    _say("oracle")
    Eo, SYMo, Lo = oracle.match(w["sym"], 16)
    _check(E, SYM, L, Eo, SYMo, Lo, "repeat")
    assert Lo.max() >= 256


def _many_copies(T, K, seed, block=60, copies=25):
    """A random stream with one block copied many times: every position in
    the later copies has more earlier recurrences than a deferred record of
    the match kernel holds."""
    rng = np.random.default_rng(seed)
    x = rng.integers(0, K, T).astype(np.uint8)
    src = x[100:100 + block].copy()
    starts = np.sort(rng.choice(np.arange(300, T - block, block + 7), copies,
                                replace=False))
    for a in starts:
        x[a:a + block] = src
    return x


def test_long_repeats_deferred_answers():
    """Long repeats, whose answers the match kernel defers to the
    time-ordered pass of the record kernel: a block copied many times (more
    candidates than a deferred record holds), nested copies (where the
    extension from the previous position fails), a length that is not a
    multiple of 4 and an alphabet above 16 (the record kernel's other
    variants).  Streams longer than the union of the large LDS plan holds
    destinations for (T > 39728) take the pass over the retrieval kernel's
    whole LDS when K <= 16 and T is a multiple of 4, else the separate
    kernel."""
    for T, K in ((8192, 16), (5001, 16), (8192, 40), (5001, 200), (65536, 16),
                 (50000, 16), (50001, 16), (65536, 40)):
        rows = [_many_copies(T, K, 11), _many_copies(T, K, 12, block=200, copies=12),
                synth.planted_copies(T, K, 13, gap_mean=50, len_lo=64, len_hi=400),
                synth.planted_copies(T, K, 14, gap_mean=20, len_lo=20, len_hi=100)]
        sym = np.stack(rows).astype(np.uint8)
        _say(f"deferred answers T={T} K={K}")
        _run_symbols(sym, K, f"deferred T={T} K={K}")


def test_long_workload_with_gather():
    _say("generating long workload")
    w = synth.long()
    H, V = w["H"], w["V"]
    Hd, Vd = _dev(H), _dev(V)
    _say("gpu")
    E, SYM, L, syms = rosa.match(Hd, M=4, want_symbols=True)
    out = torch.empty_like(Vd)
    rosa.rosa_gather(Vd, 4, E, out)
    torch.cuda.synchronize()
    _say("oracle")
    so = oracle.discretize_bf16(H, 4)
    assert np.array_equal(syms.cpu().numpy(), so)
    Eo, SYMo, Lo = oracle.match(so, 16)
    _check(E, SYM, L, Eo, SYMo, Lo, "long")
    oo = oracle.gather(V, Eo, 4)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), oo)
    # as the benchmark's pipelined steps run it: each half of the channels
    # (a strided view of H) discretised alone into 16-byte aligned symbol
    # rows, which the retrieval kernel reads itself
    _say("halves through rosa_discretize")
    S, T = so.shape
    Dh = H.shape[2] // 2
    for half, sl in ((0, slice(0, Dh)), (1, slice(Dh, 2 * Dh))):
        sy = torch.empty((S // 2, T), dtype=torch.uint8, device=DEV)
        rosa.rosa_discretize(rosa.bf16_input(Hd[:, :, sl], 4), sy)
        ws = torch.empty(rosa.rosa_match_workspace_bytes(S // 2, T, 16),
                         dtype=torch.uint8, device=DEV)
        E2, SYM2, L2, _ = rosa.match(sy, K=16, ws=ws)
        assert rosa.rosa_match_status(ws) == rosa.ROSA_OK
        rows = slice(half * S // 2, (half + 1) * S // 2)
        assert np.array_equal(sy.cpu().numpy(), so[rows])
        _check(E2, SYM2, L2, Eo[rows], SYMo[rows], Lo[rows], f"long half {half}")


def test_gather_random_destinations():
    rng = np.random.default_rng(9)
    for (B, T, D, M) in ((2, 700, 48, 4), (1, 130, 30, 3), (3, 64, 16, 8)):
        V = rng.integers(0, 65536, size=(B, T, D), dtype=np.uint16)
        S = B * D // M
        E = np.empty((S, T), dtype=np.int32)
        for t in range(T):
            E[:, t] = rng.integers(-1, t, size=S) if t > 0 else -1
        out = torch.empty((B, T, D), dtype=torch.int16, device=DEV)
        rosa.rosa_gather(_dev(V), M, _dev(E), out)
        assert np.array_equal(out.cpu().numpy().view(np.uint16),
                              oracle.gather(V, E, M))


def test_launch_geometry_independence():
    # the same streams inside different batches give the same rows
    rng = np.random.default_rng(10)
    sym = rng.integers(0, 16, size=(9, 5000), dtype=np.uint8)
    E_all = rosa.match(_dev(sym), K=16)[0].cpu().numpy()
    perm = rng.permutation(9)
    E_perm = rosa.match(_dev(sym[perm]), K=16)[0].cpu().numpy()
    assert np.array_equal(E_perm, E_all[perm])
    E_one = rosa.match(_dev(sym[3:4]), K=16)[0].cpu().numpy()
    assert np.array_equal(E_one[0], E_all[3])


@pytest.mark.parametrize("B,T,D,M,pad", [(1, 3000, 1024, 4, 0), (1, 3000, 1024, 4, 64),
                                         (1, 2000, 1024, 8, 0), (2, 900, 96, 3, 5)])
def test_gather_row_pitch(B, T, D, M, pad):
    """The value gather on V rows stored at a pitch of D + pad elements: a
    pitch that is a multiple of 2 KiB (32-route groups) and ones that are not
    (16-route groups), with and without the 8-byte vector path."""
    rng = np.random.default_rng(11 + pad + M)
    V = rng.integers(0, 65536, size=(B, T, D), dtype=np.uint16)
    S = B * D // M
    E = np.empty((S, T), dtype=np.int32)
    for t in range(T):
        E[:, t] = rng.integers(-1, t, size=S) if t > 0 else -1
    Vbuf = torch.zeros((B, T, D + pad), dtype=torch.int16, device=DEV)
    Vbuf[:, :, :D] = _dev(V.view(np.int16))
    out = torch.empty((B, T, D), dtype=torch.int16, device=DEV)
    _say(f"gather pitch B={B} T={T} D={D} M={M} pad={pad}")
    rosa.rosa_gather(Vbuf[:, :, :D], M, _dev(E), out)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), oracle.gather(V, E, M))


@pytest.mark.parametrize("B,T,D,pad,e_off", [(2, 1001, 80, 0, 0), (1, 1000, 1024, 0, 1),
                                             (3, 515, 1024, 0, 0), (1, 4109, 512, 64, 0),
                                             (1, 129, 64, 0, 3)])
def test_gather_wave_path_edges(B, T, D, pad, e_off):
    """The 8-byte (M = 4) gather: positions not a multiple of its 128-position
    chunk or of 4 (E then read one value at a time), a last route group of
    fewer than 16 routes, several batch rows, an E buffer not 16-byte aligned,
    pitches that alias (two groups per XCD) and ones that do not."""
    M = 4
    rng = np.random.default_rng(1200 + T + e_off)
    V = rng.integers(0, 65536, size=(B, T, D), dtype=np.uint16)
    S = B * D // M
    E = np.empty((S, T), dtype=np.int32)
    for t in range(T):
        E[:, t] = rng.integers(-1, t, size=S) if t > 0 else -1
    Vbuf = torch.zeros((B, T, D + pad), dtype=torch.int16, device=DEV)
    Vbuf[:, :, :D] = _dev(V.view(np.int16))
    flat = torch.empty(S * T + e_off, dtype=torch.int32, device=DEV)
    Ed = flat[e_off:].view(S, T)
    Ed.copy_(_dev(E))
    out = torch.empty((B, T, D), dtype=torch.int16, device=DEV)
    _say(f"gather wave path B={B} T={T} D={D} pad={pad} e_off={e_off}")
    rosa.rosa_gather(Vbuf[:, :, :D], M, Ed, out)
    assert np.array_equal(out.cpu().numpy().view(np.uint16), oracle.gather(V, E, M))
