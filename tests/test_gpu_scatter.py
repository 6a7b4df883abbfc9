"""GPU parity of rosa_scatter_grad (destination-scatter gradient, the
transpose of the value gather) through the C-ABI against the CPU oracle:
bit-exact float32 results (both sides sum over t in increasing order in
double precision and round once).  Cases: destinations from real matches,
many time steps per destination (the wave path), out-of-range entries,
padded rows, ragged shapes and the long workload at full size."""
import numpy as np
import pytest
import torch

import oracle
from online_suffix_automaton_amd import rosa, synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _run(theta, E, M, ldt_pad=0, ldg_pad=0):
    B, T, D = theta.shape
    if ldt_pad:
        big = torch.zeros((B, T, D + ldt_pad), dtype=torch.float32, device=DEV)
        big[:, :, :D] = torch.from_numpy(theta).to(DEV)
        th = big[:, :, :D]
    else:
        th = torch.from_numpy(theta).to(DEV)
    Gbig = torch.full((B, T, D + ldg_pad), 7.0, dtype=torch.float32, device=DEV)
    G = Gbig[:, :, :D]
    rosa.rosa_scatter_grad(th, M, torch.from_numpy(E).to(DEV), G)
    torch.cuda.synchronize()
    if ldg_pad:
        assert torch.all(Gbig[:, :, D:] == 7.0), "padding written"
    return G.cpu().numpy()


def _compare(got, want, what):
    if not np.array_equal(got.view(np.uint32), want.view(np.uint32)):
        bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} values differ, first {i}: "
                             f"gpu {got[i]!r} oracle {want[i]!r}")


@pytest.mark.parametrize("B,T,D,M", [(1, 300, 8, 1), (2, 1000, 64, 4),
                                     (3, 517, 24, 2), (1, 2048, 128, 8),
                                     (2, 777, 12, 3)])
def test_scatter_random(B, T, D, M):
    _say(f"scatter B={B} T={T} D={D} M={M}")
    rng = np.random.default_rng(B * 1000 + T + M)
    S = B * D // M
    K = min(1 << M, 16)
    x = rng.integers(0, K, (S, T)).astype(np.uint8)
    E, _, _ = oracle.match(x, K)
    theta = rng.standard_normal((B, T, D)).astype(np.float32)
    _compare(_run(theta, E, M), oracle.scatter_grad(theta, E, M), "random")


def test_scatter_many_per_destination():
    """Destinations read by up to T-1 time steps (more than 64 goes to the
    one-wave-per-destination path); large and small magnitudes mixed so
    that the summation order and precision show."""
    rng = np.random.default_rng(3)
    B, T, D, M = 1, 5000, 16, 4
    S = D // M
    E = np.full((S, T), -1, np.int32)
    E[0, 1:] = 0                               # all of stream 0 -> row 1
    E[1, 1:] = rng.integers(0, 3, T - 1)       # three destinations
    E[2, 1:] = rng.integers(-1, 100, T - 1)    # about 50 per destination
    E[3, 1:] = np.arange(T - 1)                # one per destination
    theta = (rng.standard_normal((B, T, D)) *
             10.0 ** rng.integers(-6, 7, (B, T, D))).astype(np.float32)
    _compare(_run(theta, E, M), oracle.scatter_grad(theta, E, M), "many")


@pytest.mark.parametrize("first", [7, -1, 65534])
def test_scatter_every_step_to_one_row_at_65536(first):
    """T = 65536 with (nearly) every time step, t = 0 included, pointing at
    one row: a count of 65536 would not fit the grouping kernel's 16-bit
    counters, which therefore leave t = 0 to the sum.  Stream 0 sends every
    t > 0 to row 8 and t = 0 to row E[0] + 1; stream 1 sends t = 0 to a row
    of its own; stream 2 sends every t > 0 to row 1 (65535 steps); stream 3
    is random, out-of-range entries included."""
    B, T, D, M = 1, 65536, 16, 4
    S = D // M
    rng = np.random.default_rng(11)
    E = np.full((S, T), 7, np.int32)
    E[0, 0] = first
    E[1, 0] = 100
    E[2, 0] = -1
    E[2, 1:] = 0
    E[3, :] = rng.integers(-2, T, T)
    theta = rng.standard_normal((B, T, D)).astype(np.float32)
    _compare(_run(theta, E, M), oracle.scatter_grad(theta, E, M),
             f"one row at 65536 (E[0] = {first})")


@pytest.mark.parametrize("T", [301, 300])
def test_scatter_out_of_range_and_padding(T):
    """Destinations outside [0, T-1) are ignored; T = 300 takes the grouping
    kernel's 16-byte destination loads, T = 301 the one-by-one path."""
    rng = np.random.default_rng(4 + T)
    B, D, M = 2, 32, 4
    S = B * D // M
    E = rng.integers(-5, T + 5, (S, T)).astype(np.int32)
    theta = rng.standard_normal((B, T, D)).astype(np.float32)
    _compare(_run(theta, E, M, ldt_pad=5, ldg_pad=3),
             oracle.scatter_grad(theta, E, M), "range/padding")


@pytest.mark.parametrize("T", [65536, 70001])
def test_scatter_stream_length_limits(T):
    """The longest streams counted in LDS (65536) and longer ones, which
    take the counting kernels with counters in HBM."""
    rng = np.random.default_rng(T)
    B, D, M = 1, 8, 4
    S = D // M
    E = rng.integers(-1, T - 1, (S, T)).astype(np.int32)
    E[1, : T // 2] = 7          # one destination read by half the stream
    theta = rng.standard_normal((B, T, D)).astype(np.float32)
    _compare(_run(theta, E, M), oracle.scatter_grad(theta, E, M), f"T={T}")


def test_scatter_deterministic():
    rng = np.random.default_rng(5)
    B, T, D, M = 1, 4096, 256, 4
    S = D // M
    E = rng.integers(-1, 40, (S, T)).astype(np.int32)
    theta = rng.standard_normal((B, T, D)).astype(np.float32)
    a = _run(theta, E, M)
    b = _run(theta, E, M)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_scatter_long_workload():
    """Full size: the long workload's destinations (512 streams x 65536,
    from rosa_match on the device) and an upstream gradient
    theta [1, 65536, 2048] float32 N(0,1)."""
    _say("scatter long: generating")
    w = synth.long(with_v=False)
    Hd = torch.from_numpy(w["H"].view(np.int16)).to(DEV)
    E, _, _, _ = rosa.match(Hd, M=4, want_len=False)
    del Hd
    theta = np.random.default_rng(45).standard_normal((1, 65536, 2048),
                                                      dtype=np.float32)
    _say("gpu")
    G = torch.empty((1, 65536, 2048), dtype=torch.float32, device=DEV)
    rosa.rosa_scatter_grad(torch.from_numpy(theta).to(DEV), 4, E, G)
    torch.cuda.synchronize()
    _say("oracle")
    want = oracle.scatter_grad(theta, E.cpu().numpy(), 4)
    _compare(G.cpu().numpy(), want, "long")


@pytest.mark.parametrize("pad", [0, 32, 3])
def test_scatter_theta_row_pitch(pad):
    """The scatter with theta rows at a pitch of D + pad floats (a pitch that
    is a multiple of 2 KiB and ones that are not) equals the oracle."""
    rng = np.random.default_rng(20 + pad)
    B, T, D, M = 1, 3000, 512, 4
    S = B * D // M
    theta = rng.standard_normal((B, T, D)).astype(np.float32)
    E = np.empty((S, T), dtype=np.int32)
    for t in range(T):
        E[:, t] = rng.integers(-1, t, size=S) if t > 0 else -1
    tb = torch.zeros((B, T, D + pad), dtype=torch.float32, device=DEV)
    tb[:, :, :D] = torch.from_numpy(theta).to(DEV)
    G = torch.empty((B, T, D), dtype=torch.float32, device=DEV)
    rosa.rosa_scatter_grad(tb[:, :, :D], M, torch.from_numpy(E).to(DEV), G)
    torch.cuda.synchronize()
    assert np.array_equal(G.cpu().numpy(), oracle.scatter_grad(theta, E, M))
