"""Plain, slow, obviously-correct CPU oracle for the theta-bundle reconstruction.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (the HIP library and its Python binding) never imports, links or
calls it, and this package imports nothing from the product path.

Everything is numpy float64 on the CPU.  Inputs are the exact bf16 / fp32 values
handed to the GPU, converted exactly to float64.  Each function cites the page
passage it follows:

* ``recon``     -- the reconstruction identity, the effective weight and the
                   fused Q/K/V and gate/up dispatches
                   ("How attnquant works" §The reconstruction identity;
                   "Execution paths" §Precompute-outside and §The GEMM formulation).
* ``rounding``  -- single round-to-nearest-even of an fp64 result onto the bf16 /
                   fp32 / E4M3 / E2M1 grids, written from the formats' definitions.
* ``fp4``       -- the block-16 FP4 container
                   ("Internals and extension" §Nvfp4Spec), the quantisation
                   recipe read into it, and the product of activations with the
                   dequantised weight (the FP4 decode GEMV).  PARITY UNPINNED BY THE PAGES for the
                   recipe's constants and tie rules: the pages give only the
                   container; the recipe is pinned by self-consistency, exact
                   brute force and the format tables.
* ``decompose`` -- the analytic decomposition: least-squares scale, full and
                   randomized truncated SVD, band mean
                   ("How attnquant works" §How the decomposition produces s, U, and V,
                   §The passthrough operating point).
"""

from .recon import recon_linear, recon_fused, recon_blockdiag, materialize
from .rounding import rne_bf16, rne_f32, rn_f32_exact
from .fp4 import (E2M1_VALUES, e2m1_decode, e4m3fn_decode, e4m3fn_encode_rne_sat,
                  e2m1_rne_sat, fp4_pack, fp4_unpack, fp4_linear, global_scale, FP4_BLOCK)
from .decompose import (lsq_row_scale, decompose, band_of_layer, band_means, randomized_svd,
                        decompose_randomized, FULL_SVD_MAX_MIN_DIM)

__all__ = [
    "recon_linear", "recon_fused", "recon_blockdiag", "materialize",
    "rne_bf16", "rne_f32", "rn_f32_exact",
    "E2M1_VALUES", "e2m1_decode", "e4m3fn_decode", "e4m3fn_encode_rne_sat",
    "e2m1_rne_sat", "fp4_pack", "fp4_unpack", "fp4_linear", "global_scale", "FP4_BLOCK",
    "lsq_row_scale", "decompose", "band_of_layer", "band_means", "randomized_svd",
    "decompose_randomized", "FULL_SVD_MAX_MIN_DIM",
]
