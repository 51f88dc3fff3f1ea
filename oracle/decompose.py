"""The analytic decomposition, used only to build and check test fixtures.

Test infrastructure only (see the package docstring): the oracle of the GPU
decomposition (the library's aq_decompose, aq_band_mean) and the builder of
test fixtures.

"How attnquant works" §How the decomposition produces s, U, and V:

* each output row's scale is the least-squares fit of the shared block's row to
  the target row;
* the residual after the scaled shared block is factored by a truncated SVD, and
  ``U`` absorbs the singular values so that ``U @ Vt`` is the rank-r correction;
* ``decompose`` takes the full SVD (the pages' choice when min(out, in) <= 256
  or the oversampled probe would capture the whole matrix);
  ``decompose_randomized`` applies the pages' size rule and otherwise takes the
  randomized SVD (Halko, Martinsson and Tropp 2009) with the test matrix
  passed in.

§The passthrough operating point and the band-mean sentence define the shared
block: the mean of the weights of the layers that share it, so one layer per band
gives the layer's own weight back.
"""

import numpy as np


def lsq_row_scale(W, W0):
    """s[o] = <W[o], W0[o]> / <W0[o], W0[o]>; s[o] = 1 where W0[o] is all zeros.

    The zero-row case is not addressed by the pages (any s fits equally well);
    1 keeps the passthrough case exact.
    """
    W = np.asarray(W, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    num = np.einsum("ok,ok->o", W, W0)
    den = np.einsum("ok,ok->o", W0, W0)
    return np.where(den == 0, 1.0, num / np.where(den == 0, 1.0, den))


def decompose(W, W0, r):
    """Return ``(s, U, Vt, sigma)`` with U = U_svd[:, :r] * S[:r] and Vt = Vh[:r].

    ``sigma`` is the full singular-value vector of the residual (for checks).
    ``r == 0`` gives empty ``U`` ([N, 0]) and ``Vt`` ([0, K]).
    """
    W = np.asarray(W, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    s = lsq_row_scale(W, W0)
    resid = W - s[:, None] * W0
    Usvd, S, Vh = np.linalg.svd(resid, full_matrices=False)
    U = Usvd[:, :r] * S[:r]
    Vt = Vh[:r]
    return s, U, Vt, S


# min(out_dim, in_dim) at or below which the pages take a full SVD
FULL_SVD_MAX_MIN_DIM = 256


def randomized_svd(A, r, omega, q):
    """Rank-r truncated SVD of A [N, K] by the randomized method of Halko,
    Martinsson and Tropp (2009), as the decomposition section names it, with
    the Gaussian test matrix ``omega`` [l, K] (l = r + oversampling, rows are
    the probes) passed in.  Returns ``(U, Vt, S)`` with U = U_svd[:, :r] * S[:r]
    (U absorbs the singular values), Vt = V_svd^T[:r] and S the l singular
    values of the projected matrix.

    The steps, in the paper's order (its Algorithm 4.4, the randomized range
    finder with q steps of subspace iteration, then Algorithm 5.1, the direct
    SVD of the projected matrix):
      Y = A Omega^T; Q = orth(Y);
      q times: Q~ = orth(A^T Q); Q = orth(A Q~);
      B = Q^T A; B = U_b diag(S) V^T; U_svd = Q U_b.
    orth() is numpy's QR (the Q factor); the SVD of B is numpy's.
    """
    A = np.asarray(A, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    if omega.ndim != 2 or omega.shape[1] != A.shape[1] or omega.shape[0] < r:
        raise ValueError(f"omega {omega.shape} must be [l >= r, K = {A.shape[1]}]")
    Y = A @ omega.T
    Q, _ = np.linalg.qr(Y)
    for _ in range(q):
        Qt, _ = np.linalg.qr(A.T @ Q)
        Q, _ = np.linalg.qr(A @ Qt)
    Bm = Q.T @ A
    Ub, S, Vh = np.linalg.svd(Bm, full_matrices=False)
    Usvd = Q @ Ub
    return Usvd[:, :r] * S[:r], Vh[:r], S


def decompose_randomized(W, W0, r, omega, q):
    """The decomposition as the pages describe it for any size: least-squares
    scale, residual, then the truncated SVD of the residual -- a full SVD when
    min(out_dim, in_dim) <= 256 or when the oversampled probe (l = omega's
    rows) would capture the whole matrix, else the randomized SVD with
    ``omega`` and q subspace iterations.  Returns ``(s, U, Vt, S)``."""
    W = np.asarray(W, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    s = lsq_row_scale(W, W0)
    resid = W - s[:, None] * W0
    N, K = resid.shape
    l = np.asarray(omega).shape[0]
    if min(N, K) <= FULL_SVD_MAX_MIN_DIM or l >= min(N, K):
        Usvd, S, Vh = np.linalg.svd(resid, full_matrices=False)
        return s, Usvd[:, :r] * S[:r], Vh[:r], S
    U, Vt, S = randomized_svd(resid, r, omega, q)
    return s, U, Vt, S


def band_of_layer(layer, num_layers, num_bands):
    """Contiguous bands: layer l belongs to band floor(l * G / L).

    The banded-sharing page is not among the pages; this is the plainest reading
    of 'banded' that makes G = L the passthrough case (one layer per band).
    """
    if not (0 < num_bands <= num_layers) or not (0 <= layer < num_layers):
        raise ValueError("need 0 < G <= L and 0 <= layer < L")
    return (layer * num_bands) // num_layers


def band_means(weights, num_bands):
    """Shared block of each band = mean of its layers' weights ([G] list)."""
    L = len(weights)
    groups = [[] for _ in range(num_bands)]
    for l, w in enumerate(weights):
        groups[band_of_layer(l, L, num_bands)].append(np.asarray(w, dtype=np.float64))
    return [np.mean(np.stack(g), axis=0) for g in groups]
