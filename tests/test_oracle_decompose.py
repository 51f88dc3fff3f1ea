"""Pins for the oracle's test-only decomposition and band map.

"How attnquant works" §How the decomposition produces s, U, and V and
§The passthrough operating point.  Least squares is checked by brute-force grid
search on exact rationals, the truncated SVD by the Eckart-Young identity, the
band map and band mean by direct enumeration.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle


def test_lsq_scale_bruteforce_grid():
    """W row = c * W0 row + e with e orthogonal to W0 row: the best scale is c,
    and a brute-force search over a grid containing c finds exactly c."""
    W0 = np.array([[1, 2, 0, -1], [3, 0, 1, 1], [0, 0, 2, -2]], dtype=np.float64)
    E = np.array([[2, -1, 5, 0], [0, 1, 1, -1], [7, -3, 1, 1]], dtype=np.float64)
    assert np.all(np.einsum("ok,ok->o", W0, E) == 0)
    c = np.array([0.75, -1.25, 2.5])
    W = c[:, None] * W0 + E
    s = oracle.lsq_row_scale(W, W0)
    grid = [Fraction(k, 64) for k in range(-256, 257)]
    for o in range(3):
        w = [Fraction(float(v)) for v in W[o]]
        w0 = [Fraction(float(v)) for v in W0[o]]
        cost = lambda sc: sum((a - sc * b) ** 2 for a, b in zip(w, w0))
        best = min(grid, key=cost)
        assert best == Fraction(c[o])
        assert s[o] == float(best)
        # residual orthogonal to the shared row (normal equation), exactly
        assert sum((a - best * b) * b for a, b in zip(w, w0)) == 0


def test_lsq_scale_zero_row_and_identity():
    W0 = np.array([[0.0, 0.0], [1.0, 2.0]])
    W = np.array([[3.0, 4.0], [1.0, 2.0]])
    assert oracle.lsq_row_scale(W, W0).tolist() == [1.0, 1.0]


def test_svd_eckart_young_and_absorbed_singular_values():
    rng = np.random.default_rng(0)
    N, K = 40, 30
    W = rng.standard_normal((N, K))
    W0 = rng.standard_normal((N, K))
    s, U, Vt, sigma = oracle.decompose(W, W0, r=6)
    resid = W - s[:, None] * W0
    err = np.linalg.norm(resid - U @ Vt) ** 2
    assert abs(err - np.sum(sigma[6:] ** 2)) <= 1e-10 * np.sum(sigma ** 2)
    # U absorbs S: column norms are the singular values; Vt rows are orthonormal
    assert np.allclose(np.linalg.norm(U, axis=0), sigma[:6], rtol=1e-12)
    assert np.allclose(Vt @ Vt.T, np.eye(6), atol=1e-12)
    # full rank -> exact
    s2, U2, Vt2, _ = oracle.decompose(W, W0, r=min(N, K))
    assert np.max(np.abs(resid - U2 @ Vt2)) < 1e-12


def test_rank_zero_gives_empty_factors():
    W = np.ones((5, 8)); W0 = np.ones((5, 8)) * 2
    s, U, Vt, _ = oracle.decompose(W, W0, r=0)
    assert U.shape == (5, 0) and Vt.shape == (0, 8)
    assert np.array_equal(s, np.full(5, 0.5))


def test_band_map_contiguous():
    assert [oracle.band_of_layer(l, 26, 13) for l in range(26)] == [l // 2 for l in range(26)]
    assert [oracle.band_of_layer(l, 8, 4) for l in range(8)] == [0, 0, 1, 1, 2, 2, 3, 3]
    assert [oracle.band_of_layer(l, 7, 7) for l in range(7)] == list(range(7))
    assert [oracle.band_of_layer(l, 5, 1) for l in range(5)] == [0] * 5


def test_band_mean_and_passthrough():
    rng = np.random.default_rng(2)
    Ws = [rng.integers(-8, 8, size=(6, 10)).astype(np.float64) for _ in range(4)]
    means = oracle.band_means(Ws, 2)
    assert np.array_equal(means[0], (Ws[0] + Ws[1]) / 2)
    assert np.array_equal(means[1], (Ws[2] + Ws[3]) / 2)
    # G = L: each band's shared block is the layer's own weight -> exact rebuild
    own = oracle.band_means(Ws, 4)
    x = rng.integers(-3, 4, size=(3, 10)).astype(np.float64)
    for l in range(4):
        assert np.array_equal(own[l], Ws[l])
        s, U, Vt, _ = oracle.decompose(Ws[l], own[l], r=3)
        assert np.array_equal(oracle.recon_linear(x, own[l], s, U, Vt), x @ Ws[l].T)


# ------------------------------------------------------------- randomized SVD

def _gapped(N, K, r, seed, tail=1e-6, top=2.0):
    """A [N, K] with singular values top .. 1 (geometric) for the first r and
    `tail` times smaller after, from random orthonormal factors (numpy's QR)."""
    rng = np.random.default_rng(seed)
    m = min(N, K)
    P, _ = np.linalg.qr(rng.standard_normal((N, m)))
    R, _ = np.linalg.qr(rng.standard_normal((K, m)))
    sig = np.concatenate([np.geomspace(top, 1.0, r), tail * np.linspace(1.0, 0.5, m - r)])
    return (P * sig) @ R.T, sig


def test_randomized_svd_exact_rank_is_exact():
    """A matrix of rank <= l is captured exactly: U Vt = A (any q), and equals
    the full SVD's truncation."""
    rng = np.random.default_rng(1)
    N, K, k = 300, 280, 6
    A = rng.standard_normal((N, k)) @ rng.standard_normal((k, K))
    om = rng.standard_normal((16, K))
    for q in (0, 2):
        U, Vt, S = oracle.randomized_svd(A, 6, om, q)
        assert np.max(np.abs(U @ Vt - A)) <= 1e-10 * np.max(np.abs(A))
    Uf, Sf, Vf = np.linalg.svd(A)
    assert np.allclose(S[:6], Sf[:6], rtol=1e-12)


def test_randomized_svd_matches_truncation_on_gapped_spectrum():
    """With a clear gap after r, the randomized truncation is the truncated SVD
    to within the tail (Halko et al.'s bound: error of the order of
    sigma_{r+1})."""
    N, K, r = 400, 350, 8
    A, sig = _gapped(N, K, r, 2)
    om = np.random.default_rng(3).standard_normal((r + 10, K))
    U, Vt, S = oracle.randomized_svd(A, r, om, 2)
    Uf, Sf, Vhf = np.linalg.svd(A, full_matrices=False)
    Ar = (Uf[:, :r] * Sf[:r]) @ Vhf[:r]
    assert np.linalg.norm(U @ Vt - Ar, 2) <= 10 * sig[r]
    assert np.allclose(S[:r], sig[:r], rtol=1e-10)


def test_randomized_svd_factor_structure_and_eckart_young():
    """U = U_svd S (orthogonal columns of norms S), Vt orthonormal rows, the
    error never below the Eckart-Young optimum, and subspace iteration brings it
    to the optimum on a slowly decaying spectrum (q = 6 beats q = 0)."""
    rng = np.random.default_rng(4)
    N, K, r = 260, 300, 10
    A = rng.standard_normal((N, K)) * np.exp(-np.arange(K) / 40.0)[None, :]
    sig = np.linalg.svd(A, compute_uv=False)
    om = rng.standard_normal((r + 10, K))
    errs = []
    for q in (0, 6):
        U, Vt, S = oracle.randomized_svd(A, r, om, q)
        assert np.allclose(Vt @ Vt.T, np.eye(r), atol=1e-12)
        G = U.T @ U
        assert np.allclose(np.diag(G), S[:r] ** 2, rtol=1e-10)
        assert np.max(np.abs(G - np.diag(np.diag(G)))) <= 1e-10 * S[0] ** 2
        e = np.linalg.norm(A - U @ Vt) ** 2
        assert e >= np.sum(sig[r:] ** 2) * (1 - 1e-12)
        errs.append(e)
    assert errs[1] < errs[0]
    assert errs[1] <= np.sum(sig[r:] ** 2) * (1 + 1e-3)


def test_decompose_randomized_size_rule():
    """min(out, in) <= 256, or a probe as wide as the matrix: the full SVD
    (identical to oracle.decompose); beyond, the randomized SVD."""
    rng = np.random.default_rng(5)
    W0 = rng.standard_normal((200, 300))
    W = 1.1 * W0 + rng.standard_normal((200, 300)) * 0.1
    om = rng.standard_normal((14, 300))
    s, U, Vt, S = oracle.decompose_randomized(W, W0, 4, om, 2)
    s2, U2, Vt2, S2 = oracle.decompose(W, W0, 4)
    assert np.array_equal(s, s2) and np.allclose(U @ Vt, U2 @ Vt2, rtol=0, atol=1e-13)
    W0b = rng.standard_normal((300, 320))
    Wb = 0.9 * W0b + rng.standard_normal((300, 320)) * 0.1
    om2 = rng.standard_normal((300, 320))                          # probe covers min(N, K)
    sb, Ub, Vtb, _ = oracle.decompose_randomized(Wb, W0b, 5, om2, 1)
    sf, Uf, Vtf, _ = oracle.decompose(Wb, W0b, 5)
    assert np.allclose(Ub @ Vtb, Uf @ Vtf, atol=1e-12)
    om3 = rng.standard_normal((15, 320))                           # randomized branch
    sr, Ur, Vtr, _ = oracle.decompose_randomized(Wb, W0b, 5, om3, 2)
    resid = Wb - sr[:, None] * W0b
    U4, Vt4, _ = oracle.randomized_svd(resid, 5, om3, 2)
    assert np.array_equal(Ur @ Vtr, U4 @ Vt4)


def test_randomized_pins_catch_planted_mistakes():
    """Copies of the randomized SVD with plausible mistakes each fail a pin:
    S not absorbed into U, V's columns instead of rows, no re-orthonormalisation
    in the subspace iteration (the basis collapses onto the top direction),
    the probe applied to A^T."""
    N, K, r = 320, 300, 6
    # a wide spread of the leading singular values (1e4 .. 1): without
    # re-orthonormalisation, q = 8 subspace steps raise it to the 17th power
    # and the basis collapses onto the top directions in float64
    A, sig = _gapped(N, K, r, 6, tail=1e-3, top=1e4)
    om = np.random.default_rng(8).standard_normal((r + 10, K))

    def no_absorb(A, r, om, q):
        U, Vt, S = oracle.randomized_svd(A, r, om, q)
        return U / S[:r], Vt, S

    def vh_columns(A, r, om, q):
        U, Vt, S = oracle.randomized_svd(A, r, om, q)
        Q, _ = np.linalg.qr(A @ om.T)
        _, _, Vh = np.linalg.svd(Q.T @ A, full_matrices=False)
        return U, Vh[:, :r].T if Vh.shape[1] >= r else Vt, S

    def no_reorth(A, r, om, q):
        Y = A @ om.T
        for _ in range(q):
            Y = A @ (A.T @ Y)
        Q, _ = np.linalg.qr(Y)
        Ub, S, Vh = np.linalg.svd(Q.T @ A, full_matrices=False)
        return (Q @ Ub)[:, :r] * S[:r], Vh[:r], S

    def pins_pass(fn):
        try:
            U, Vt, S = fn(A, r, om, 8)
            Uf, Sf, Vhf = np.linalg.svd(A, full_matrices=False)
            ok = np.linalg.norm(U @ Vt - (Uf[:, :r] * Sf[:r]) @ Vhf[:r], 2) <= 10 * Sf[r]
            ok &= np.allclose(np.linalg.norm(U, axis=0), S[:r], rtol=1e-8)
            ok &= np.allclose(Vt @ Vt.T, np.eye(r), atol=1e-10)
            return bool(ok)
        except (ValueError, np.linalg.LinAlgError):
            return False

    assert pins_pass(oracle.randomized_svd)
    for bad in (no_absorb, vh_columns, no_reorth):
        assert not pins_pass(bad), bad.__name__
    # the probe on the wrong side of a non-square matrix breaks the shapes
    with pytest.raises(ValueError):
        oracle.randomized_svd(A, r, np.zeros((r + 10, N)), 1)
