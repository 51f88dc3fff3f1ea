"""Shared helpers for the GPU parity tests: upload the seeded inputs, download
results, compare against the oracle with the stated tolerances."""

import numpy as np
import torch

import oracle

# Tolerances: max|y_gpu - y_ref| / max|y_ref| (the spec bar) ...
TOL_BF16 = 1e-2
TOL_F32 = 1e-5
# ... and the tighter bound that the arithmetic itself allows for bf16: one
# round-to-nearest of y to bf16 (bf16 keeps 8 significant bits, so the unit
# roundoff is 2^-8 = 3.91e-3 of |y| <= max|y|), fp32 accumulation (~1e-6 of
# max|y| on these inputs) and the bf16 rounding of the rank-r activation t used
# as an MFMA operand (2^-8 of the low-rank term, which is itself ~5% of max|y|
# on these inputs, so ~2e-4 at most and far less in practice).  4e-3 leaves
# ~1e-4 above the output rounding for the rest; a kernel that loses more than
# that fails here well before it reaches the 1e-2 bar.
TOL_BF16_DERIVED = 4e-3

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return torch.device("cuda", 0)


def up(a, dtype, device=None):
    """numpy float32 array (values exact in `dtype`) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(device or dev()).to(TORCH_DT[dtype])


def down(t):
    return t.float().cpu().numpy().astype(np.float64)


def bundle_up(bd, dtype, device=None):
    return tuple(up(bd[k], dtype, device) for k in ("W0", "s", "U", "Vt"))


def bundle_np(bd):
    return tuple(np.asarray(bd[k], dtype=np.float64) for k in ("W0", "s", "U", "Vt"))


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    if scale == 0.0:
        return 0.0 if err == 0.0 else np.inf
    return err / scale


def assert_parity(got, ref, dtype, what=""):
    e = rel_err(got, ref)
    if dtype == "f32":
        assert e <= TOL_F32, f"{what}: rel err {e:.3e} > {TOL_F32}"
    else:
        assert e <= TOL_BF16, f"{what}: rel err {e:.3e} > {TOL_BF16}"
        assert e <= TOL_BF16_DERIVED, f"{what}: rel err {e:.3e} > derived bound {TOL_BF16_DERIVED}"
    return e


def sub_bundle(bd, cols):
    """The bundle (an inputs.bundle dict) restricted to output rows `cols`, as
    float64: the identity is separable in the output index, so
    oracle(sub_bundle)[:, i] == oracle(full)[:, cols[i]]."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    return (f(bd["W0"][cols]), f(bd["s"][cols]), f(bd["U"][cols]), f(bd["Vt"]))
