"""Pins for the oracle's test-only decomposition and band map.

"How attnquant works" §How the decomposition produces s, U, and V and
§The passthrough operating point.  Least squares is checked by brute-force grid
search on exact rationals, the truncated SVD by the Eckart-Young identity, the
band map and band mean by direct enumeration.
"""

from fractions import Fraction

import numpy as np

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
