"""Pins for the oracle's reconstruction identity, effective weight and fused forms.

Each pin checks the oracle against something other than itself: a hand-worked
golden case, exact integer brute force that builds the dense weight element by
element, the pages' invariants (factored == materialised, r = 0, passthrough,
block-diagonal fusion), and linearity.  ``test_pins_catch_planted_mistakes``
plants plausible mistakes in a copy of the oracle and checks that the pins fail.
"""

import json
import os
import random

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _int_bundle(rng, N, K, r, lo=-3, hi=4):
    W0 = rng.integers(lo, hi, size=(N, K)).astype(np.float64)
    s = rng.integers(lo, hi, size=(N,)).astype(np.float64)
    U = rng.integers(lo, hi, size=(N, r)).astype(np.float64)
    Vt = rng.integers(lo, hi, size=(r, K)).astype(np.float64)
    return W0, s, U, Vt


def _brute_dense(W0, s, U, Vt):
    """Dense weight element by element with Python integers (exact)."""
    N, K = W0.shape
    r = U.shape[1]
    W = [[int(s[n]) * int(W0[n][k]) + sum(int(U[n][j]) * int(Vt[j][k]) for j in range(r))
          for k in range(K)] for n in range(N)]
    return W


def _brute_apply(W, x):
    return [[sum(W[n][k] * int(x[m][k]) for k in range(len(W[0]))) for n in range(len(W))]
            for m in range(len(x))]


# --------------------------------------------------------------------------- pins

def pin_hand_case(recon_linear, materialize):
    g = _golden("hand_recon_2x3.json")
    W0, s, U, Vt, x = (np.array(g[k], dtype=np.float64) for k in ("W0", "s", "U", "Vt", "x"))
    y = recon_linear(x, W0, s, U, Vt)
    assert np.array_equal(y, np.array(g["y"], dtype=np.float64))
    assert np.array_equal(materialize(W0, s, U, Vt), np.array(g["W_eff"], dtype=np.float64))


def pin_integer_bruteforce(recon_linear, materialize, trials=60):
    rng = np.random.default_rng(1234)
    for _ in range(trials):
        N, K, r, M = (int(v) for v in rng.integers(1, 6, size=4))
        r = int(rng.integers(0, 4))
        W0, s, U, Vt = _int_bundle(rng, N, K, r)
        x = rng.integers(-3, 4, size=(M, K)).astype(np.float64)
        W = _brute_dense(W0, s, U, Vt)
        assert np.array_equal(materialize(W0, s, U, Vt), np.array(W, dtype=np.float64))
        assert np.array_equal(recon_linear(x, W0, s, U, Vt),
                              np.array(_brute_apply(W, x), dtype=np.float64))


def pin_rank0(recon_linear, trials=30):
    rng = np.random.default_rng(99)
    for _ in range(trials):
        N, K, M = (int(v) for v in rng.integers(1, 7, size=3))
        W0, s, U, Vt = _int_bundle(rng, N, K, 0)
        x = rng.integers(-4, 5, size=(M, K)).astype(np.float64)
        want = [[int(s[n]) * sum(int(W0[n][k]) * int(x[m][k]) for k in range(K))
                 for n in range(N)] for m in range(M)]
        assert np.array_equal(recon_linear(x, W0, s, U, Vt), np.array(want, dtype=np.float64))


def pin_factored_equals_materialised(recon_linear, materialize):
    rng = np.random.default_rng(7)
    for (N, K, r, M) in [(37, 53, 5, 9), (64, 32, 16, 3), (5, 80, 0, 4)]:
        W0 = rng.standard_normal((N, K)) / np.sqrt(K)
        s = rng.uniform(0.9, 1.1, N)
        U = rng.standard_normal((N, r)) * 0.3
        Vt = rng.standard_normal((r, K)) * 0.3
        x = rng.standard_normal((M, K))
        y = recon_linear(x, W0, s, U, Vt)
        y2 = x @ materialize(W0, s, U, Vt).T
        assert np.max(np.abs(y - y2)) <= 1e-12 * max(1.0, np.max(np.abs(y2)))


def pin_linearity(recon_linear):
    rng = np.random.default_rng(11)
    N, K, r, M = 19, 23, 4, 3
    W0 = rng.standard_normal((N, K)); s = rng.standard_normal(N)
    U = rng.standard_normal((N, r)); Vt = rng.standard_normal((r, K))
    x1 = rng.standard_normal((M, K)); x2 = rng.standard_normal((M, K))
    a, b = 1.75, -0.5
    lhs = recon_linear(a * x1 + b * x2, W0, s, U, Vt)
    rhs = a * recon_linear(x1, W0, s, U, Vt) + b * recon_linear(x2, W0, s, U, Vt)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))


PINS = (pin_hand_case, pin_integer_bruteforce, pin_rank0,
        pin_factored_equals_materialised, pin_linearity)


def _run_pins(recon_linear, materialize):
    failures = []
    for pin in PINS:
        kwargs = {}
        if "materialize" in pin.__code__.co_varnames[:pin.__code__.co_argcount]:
            kwargs["materialize"] = materialize
        try:
            pin(recon_linear, **kwargs)
        except AssertionError:
            failures.append(pin.__name__)
    return failures


# --------------------------------------------------------------------------- tests

def test_hand_case():
    pin_hand_case(oracle.recon_linear, oracle.materialize)


def test_integer_bruteforce():
    pin_integer_bruteforce(oracle.recon_linear, oracle.materialize)


def test_rank0_is_scaled_shared_block():
    pin_rank0(oracle.recon_linear)


def test_factored_equals_materialised():
    pin_factored_equals_materialised(oracle.recon_linear, oracle.materialize)


def test_linearity():
    pin_linearity(oracle.recon_linear)


def test_passthrough_reproduces_weight_exactly():
    """G = L: W0 is the layer's own weight, s = 1, U V^T = 0, output = x W^T bit for bit."""
    rng = np.random.default_rng(5)
    W = rng.standard_normal((24, 40)).astype(np.float32).astype(np.float64)
    x = rng.standard_normal((6, 40)).astype(np.float32).astype(np.float64)
    s, U, Vt, sigma = oracle.decompose(W, W, r=4)
    assert np.array_equal(s, np.ones(24))
    assert np.array_equal(U @ Vt, np.zeros((24, 40)))
    assert np.array_equal(oracle.recon_linear(x, W, s, U, Vt), np.matmul(x, W.T))
    assert np.array_equal(oracle.materialize(W, s, U, Vt), W)


def test_fused_equals_concat_and_blockdiag():
    rng = np.random.default_rng(3)
    K, M = 48, 5
    shapes = [(32, 6), (8, 6), (8, 6)]
    bundles = []
    for N, r in shapes:
        bundles.append((rng.standard_normal((N, K)), rng.uniform(0.9, 1.1, N),
                        rng.standard_normal((N, r)), rng.standard_normal((r, K))))
    x = rng.standard_normal((M, K))
    fused = oracle.recon_fused(x, bundles)
    bd = oracle.recon_blockdiag(x, bundles)
    assert fused.shape == (M, 48)
    assert np.max(np.abs(fused - bd)) <= 1e-12 * np.max(np.abs(bd))
    col = 0
    for b in bundles:
        n = b[0].shape[0]
        assert np.array_equal(fused[:, col:col + n], oracle.recon_linear(x, *b))
        col += n


def test_blockdiag_is_block_local():
    """Changing U_q moves only the q columns of the fused output."""
    rng = np.random.default_rng(4)
    K, M = 32, 3
    bundles = [(rng.standard_normal((n, K)), np.ones(n), rng.standard_normal((n, 2)),
                rng.standard_normal((2, K))) for n in (16, 4, 4)]
    base = oracle.recon_blockdiag(rng.standard_normal((M, K)) * 0 + 1, bundles)
    bumped = list(bundles)
    W0, s, U, Vt = bundles[0]
    bumped[0] = (W0, s, U + 1.0, Vt)
    moved = oracle.recon_blockdiag(np.ones((M, K)), bumped)
    assert not np.allclose(moved[:, :16], base[:, :16])
    assert np.array_equal(moved[:, 16:], base[:, 16:])


def test_shape_mismatch_raises():
    W0 = np.zeros((4, 8)); s = np.ones(4); U = np.zeros((4, 2)); Vt = np.zeros((3, 8))
    with pytest.raises(ValueError):
        oracle.recon_linear(np.zeros((1, 8)), W0, s, U, Vt)
    with pytest.raises(ValueError):
        oracle.recon_linear(np.zeros((1, 7)), W0, s, np.zeros((4, 3)), Vt)


# Plausible mistakes, each planted in a copy of the oracle's arithmetic.
def _mut_drop_scale(x, W0, s, U, Vt):
    x, W0, U, Vt = map(np.asarray, (x, W0, U, Vt))
    return x @ W0.T + (x @ Vt.T) @ U.T


def _mut_scale_after_lowrank(x, W0, s, U, Vt):
    return np.asarray(s)[None, :] * (x @ np.asarray(W0).T + (x @ np.asarray(Vt).T) @ np.asarray(U).T)


def _mut_minus_lowrank(x, W0, s, U, Vt):
    return np.asarray(s)[None, :] * (x @ np.asarray(W0).T) - (x @ np.asarray(Vt).T) @ np.asarray(U).T


def _mut_drop_lowrank(x, W0, s, U, Vt):
    return np.asarray(s)[None, :] * (x @ np.asarray(W0).T)


def _mut_scale_columns(x, W0, s, U, Vt):
    W0 = np.asarray(W0, dtype=float)
    s = np.asarray(s, dtype=float)
    K = W0.shape[1]
    sc = np.resize(s, K)               # scale along the input axis instead of rows
    return (x * sc[None, :]) @ W0.T + (x @ np.asarray(Vt).T) @ np.asarray(U).T


def _mut_mat_drop_scale(W0, s, U, Vt):
    return np.asarray(W0, dtype=float) + np.asarray(U) @ np.asarray(Vt)


def _mut_mat_scale_columns(W0, s, U, Vt):
    W0 = np.asarray(W0, dtype=float)
    return W0 * np.resize(np.asarray(s, dtype=float), W0.shape[1])[None, :] + np.asarray(U) @ np.asarray(Vt)


@pytest.mark.parametrize("recon,mat", [
    (_mut_drop_scale, oracle.materialize),
    (_mut_scale_after_lowrank, oracle.materialize),
    (_mut_minus_lowrank, oracle.materialize),
    (_mut_drop_lowrank, oracle.materialize),
    (_mut_scale_columns, oracle.materialize),
    (oracle.recon_linear, _mut_mat_drop_scale),
    (oracle.recon_linear, _mut_mat_scale_columns),
])
def test_pins_catch_planted_mistakes(recon, mat):
    assert _run_pins(recon, mat), "a planted mistake passed every pin"


def test_pins_pass_on_the_oracle():
    assert _run_pins(oracle.recon_linear, oracle.materialize) == []
