"""Pins for the destination-scatter oracle (no GPU): hand-worked examples
(tests/golden/scatter_examples.json), the adjoint identity with the pinned
gather oracle (sum theta * gather(V) = sum G * V, exact on integer values),
conservation of the total gradient, and the out-of-range destinations."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
EXAMPLES = json.load(open(os.path.join(GOLD, "scatter_examples.json")))["examples"]


@pytest.mark.parametrize("ex", EXAMPLES, ids=lambda e: e["name"])
def test_scatter_hand_examples(ex):
    theta = np.asarray(ex["theta"], np.float32)
    E = np.asarray(ex["E"], np.int32)
    G = oracle.scatter_grad(theta, E, ex["M"])
    assert G.tolist() == ex["G"]


def _bf16_of_ints(a):
    """Small integers as exact bf16 bit patterns."""
    f = a.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("M", [1, 2, 4])
def test_adjoint_of_gather(M):
    rng = np.random.default_rng(30 + M)
    B, T, D = 2, 300, 8 * M
    S = B * D // M
    x = rng.integers(0, 4, (S, T)).astype(np.uint8)
    E, _, _ = oracle.match(x, 4)
    theta = rng.integers(-50, 50, (B, T, D)).astype(np.float32)
    vint = rng.integers(-100, 100, (B, T, D))
    V = _bf16_of_ints(vint)
    g = oracle.gather(V, E, M)
    gv = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    G = oracle.scatter_grad(theta, E, M)
    lhs = float((theta.astype(np.float64) * gv).sum())
    rhs = float((G.astype(np.float64) * vint).sum())
    assert lhs == rhs


def test_total_gradient_is_conserved():
    rng = np.random.default_rng(40)
    B, T, D, M = 1, 2000, 16, 4
    S = D // M
    x = rng.integers(0, 16, (S, T)).astype(np.uint8)
    E, _, _ = oracle.match(x, 16)
    theta = rng.integers(-1000, 1000, (B, T, D)).astype(np.float32)
    G = oracle.scatter_grad(theta, E, M)
    valid = (E >= 0)                       # [S, T]
    for s in range(S):
        cols = slice(s * M, (s + 1) * M)
        want = theta[0, valid[s], cols].astype(np.float64).sum(0)
        assert np.array_equal(G[0, :, cols].astype(np.float64).sum(0), want)


def test_out_of_range_destinations_add_nothing():
    theta = np.ones((1, 4, 2), np.float32)
    E = np.array([[3, -5, 2, 7]], np.int32)   # tau = 4, -, 3, 8: only 3 in range
    G = oracle.scatter_grad(theta, E, 2)
    want = np.zeros((1, 4, 2), np.float32)
    want[0, 3] = 1
    assert np.array_equal(G, want)
