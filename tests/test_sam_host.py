"""The decode automaton's own code (csrc/rosa_sam_core.h), compiled for the
host, against the oracle: a prefix appended without last-end walks with the
last ends then set in one pass (what rosa_build does), followed by online
steps with the walk (what rosa_step does).  E and L of every stepped
position must equal the oracle's.  Streams: constant (whose walks would
cost O(T^2) in the prefix build), periodic, planted repeats and i.i.d., up
to 65,536 positions.  CPU only (hipcc builds the host program; no GPU)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("sam") / "sam_build_check")
    subprocess.check_call(
        [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17",
         "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "online_suffix_automaton_amd", "csrc"),
         os.path.join(ROOT, "tests", "host", "sam_build_check.cpp"), "-o", exe],
        stderr=subprocess.DEVNULL)
    return exe


def _run(exe, x, K, T0):
    r = subprocess.run([exe, str(K), str(T0)], input=x.astype(np.uint8).tobytes(),
                       capture_output=True, timeout=300)
    assert r.returncode == 0, r.stderr
    a = np.array(r.stdout.split(), dtype=np.int64).reshape(-1, 3)
    return a[:, 0], a[:, 1], a[:, 2]


def _streams():
    rng = np.random.default_rng(21)
    T = 65536
    yield "constant", np.zeros(T, np.uint8), 16
    yield "period 3", np.tile(np.array([1, 2, 3], np.uint8), T // 3 + 1)[:T], 16
    yield "binary iid", rng.integers(0, 2, T).astype(np.uint8), 2
    x = rng.integers(0, 16, T).astype(np.uint8)
    for _ in range(40):
        L = int(rng.integers(32, 2000))
        s0 = int(rng.integers(0, T - 2 * L))
        d0 = int(rng.integers(s0 + L, T - L))
        x[d0:d0 + L] = x[s0:s0 + L]
    yield "planted repeats", x, 16
    yield "iid K=16", rng.integers(0, 16, T).astype(np.uint8), 16
    yield "iid K=256 short", rng.integers(0, 256, 5000).astype(np.uint8), 256


@pytest.mark.parametrize("case", list(range(6)))
def test_prefix_build_then_steps_match_oracle(harness, case):
    name, x, K = list(_streams())[case]
    T = len(x)
    E, _, L = oracle.match(x[None, :], K)
    # (steps on a constant or periodic stream walk O(t) states each, so those
    # start late; the prefix build is the part under test there)
    starts = (T // 2, T - 300) if name in ("constant", "period 3") else \
        (0, 1, T // 2, T - 300)
    for T0 in starts:
        t, e, l = _run(harness, x, K, T0)
        assert np.array_equal(t, np.arange(T0, T)), name
        bad = np.nonzero((e != E[0, T0:]) | (l != L[0, T0:]))[0]
        assert bad.size == 0, (f"{name}, prefix {T0}: first difference at t = "
                               f"{T0 + bad[0]}: E {e[bad[0]]} vs {E[0, T0 + bad[0]]}, "
                               f"L {l[bad[0]]} vs {L[0, T0 + bad[0]]}")
