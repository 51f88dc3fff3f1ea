"""The analytic decomposition, used only to build and check test fixtures.

Test infrastructure only (see the package docstring).  Not part of the hot path:
the GPU library consumes a bundle, it never produces one.

"How attnquant works" §How the decomposition produces s, U, and V:

* each output row's scale is the least-squares fit of the shared block's row to
  the target row;
* the residual after the scaled shared block is factored by a truncated SVD, and
  ``U`` absorbs the singular values so that ``U @ Vt`` is the rank-r correction;
* for the sizes used here (min(out, in) <= 256) the pages fall back to a full
  SVD, which is what this module does.

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
