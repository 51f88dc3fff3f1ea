"""Reconstruction identity, effective weight and fused dispatches, in float64.

Test infrastructure only (see the package docstring).

Conventions (the plainest reading of the pages, stated once here):

* ``x`` is a batch of row vectors ``[M, K]`` (K = in_dim); outputs are ``[M, N]``
  (N = out_dim).  The pages write the identity for a column vector,
  ``y = s . (W0 x) + U (V^T x)``, and the GEMM path writes the same thing for a
  row batch, ``y = s[None, :] * (x @ W0.T) + (x @ V) @ U.T``
  ("Execution paths" §The GEMM formulation).
* ``W0`` is ``[N, K]``; ``s`` is ``[N]``, one scale per output row
  ("How attnquant works" §The theta bundle); ``U`` is ``[N, r]``.
* ``V`` is ``[K, r]`` on the pages (it multiplies ``x`` on the right); it is passed
  here transposed, ``Vt = V^T`` with shape ``[r, K]``.  ``U @ Vt`` is then the
  pages' ``U . V^T``.
* ``r = 0`` is allowed: ``U`` is ``[N, 0]`` and ``Vt`` is ``[0, K]`` and the low-rank
  term vanishes ("How attnquant works", end of §How the decomposition produces
  s, U, and V).
"""

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _check_bundle(W0, s, U, Vt):
    N, K = W0.shape
    r = U.shape[1]
    if s.shape != (N,) or U.shape != (N, r) or Vt.shape != (r, K):
        raise ValueError(f"bundle shapes disagree: W0{W0.shape} s{s.shape} U{U.shape} Vt{Vt.shape}")
    return N, K, r


def recon_linear(x, W0, s, U, Vt):
    """y = s * (x W0^T) + (x Vt^T) U^T, unrounded float64.

    "How attnquant works" §The reconstruction identity (the projection output
    rebuilt from the bundle without forming the dense matrix); row-batch form as
    in "Execution paths" §The GEMM formulation.  The product ``x @ Vt.T`` is the
    rank-r down-projection ``t``; ``t @ U.T`` is the up-projection.
    """
    x, W0, s, U, Vt = map(_f64, (x, W0, s, U, Vt))
    _check_bundle(W0, s, U, Vt)
    if x.ndim != 2 or x.shape[1] != W0.shape[1]:
        raise ValueError(f"x {x.shape} does not match W0 {W0.shape}")
    z = x @ W0.T                # shared-block term, [M, N]
    t = x @ Vt.T                # low-rank down-projection, [M, r]
    return s[None, :] * z + t @ U.T


def recon_fused(x, bundles):
    """Several projections that read the same x, outputs concatenated along N.

    ``bundles`` is a sequence of ``(W0, s, U, Vt)`` in output order: (q, k, v) for
    the attention dispatch, (gate, up) for the MLP dispatch.  "Execution paths"
    §The GEMM formulation batches Q/K/V (and gate/up) into one down-contraction
    over the concatenated blocks and one block-diagonal up-projection;
    §Precompute-outside says the stacked layers concatenate along the output
    axis.  Written here as the plain concatenation of the separate projections;
    ``recon_blockdiag`` writes the block-diagonal form and the tests check the
    two agree.
    """
    return np.concatenate([recon_linear(x, *b) for b in bundles], axis=1)


def recon_blockdiag(x, bundles):
    """The fused dispatch written literally as the pages' two GEMMs.

    One GEMM of ``x`` against the row-stacked ``[W0_q; W0_k; W0_v]`` and the
    row-stacked ``[Vt_q; Vt_k; Vt_v]``, then one GEMM of the resulting ``t`` with
    the block-diagonal ``blockdiag(U_q, U_k, U_v)`` ("Execution paths" §The GEMM
    formulation, the Q/K/V batching paragraph).  Only for small shapes: it forms
    the block-diagonal matrix explicitly.
    """
    x = _f64(x)
    W0s, ss, Us, Vts = [], [], [], []
    for (W0, s, U, Vt) in bundles:
        W0, s, U, Vt = map(_f64, (W0, s, U, Vt))
        _check_bundle(W0, s, U, Vt)
        W0s.append(W0); ss.append(s); Us.append(U); Vts.append(Vt)
    W0_cat = np.concatenate(W0s, axis=0)            # [sum N, K]
    Vt_cat = np.concatenate(Vts, axis=0)            # [sum r, K]
    s_cat = np.concatenate(ss)
    n_tot = W0_cat.shape[0]
    r_tot = Vt_cat.shape[0]
    U_bd = np.zeros((n_tot, r_tot))
    n0 = r0 = 0
    for U in Us:
        n, r = U.shape
        U_bd[n0:n0 + n, r0:r0 + r] = U
        n0 += n
        r0 += r
    down = x @ np.concatenate([W0_cat, Vt_cat], axis=0).T   # one x @ [W0^T, V]
    z, t = down[:, :n_tot], down[:, n_tot:]
    return s_cat[None, :] * z + t @ U_bd.T


def materialize(W0, s, U, Vt):
    """W_eff = diag(s) W0 + U V^T, unrounded float64, shape [N, K].

    "Execution paths" §Precompute-outside (the weight rebuilt once at load) and
    "How attnquant works" §The reconstruction identity (diag(s) scales the rows
    of W0).  Rounding to the storage dtype is a separate step
    (``oracle.rounding``).
    """
    W0, s, U, Vt = map(_f64, (W0, s, U, Vt))
    _check_bundle(W0, s, U, Vt)
    return s[:, None] * W0 + U @ Vt
