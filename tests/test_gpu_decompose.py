"""GPU parity of the decomposition (aq_band_mean, aq_decompose) against the
oracle's: the band mean bit for bit, the least-squares scale and the rank-r
product U Vt of the truncated SVD of the residual (the singular vectors
themselves are unique only up to sign), with the same Gaussian probe on both
sides.

Tolerances: both sides compute in float64; they differ in the order of their
sums and in the factorisations they use for the same mathematical steps (the
GPU: Cholesky QR twice and a Jacobi eigendecomposition of B B^T; the oracle:
Householder QR and LAPACK's SVD).  Rounding of ~1e-16, amplified by at most
sigma_1^2 / (sigma_r^2 - sigma_{r+1}^2) in the truncated subspace (the fixtures
have a clear gap after r), stays far below the 1e-9 (of max |U Vt|) checked
here; the scale is a quotient of two K-term dot products, 1e-12 relative."""

import numpy as np
import pytest
import torch

import oracle
from rank_shared_block_amd import binding as B
from rank_shared_block_amd import inputs as I
from helpers import bundle_np, bundle_up, dev, down, rel_err, up

pytestmark = pytest.mark.gpu

TOL_UV = 1e-9
TOL_S = 1e-12


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev()).to(dtype)


def _weights(N, K, r, layer, dtype="bf16", band=0, family="q"):
    """A trained-like weight with a low-rank perturbation of rank r (r / 2
    cosine waves) and its band's shared block."""
    W = I.trained_weight("decompose", layer, family, K, N, dtype, band=band, waves=max(1, r // 2))
    W0 = I.bundle("decompose", layer, family, K, N, 0, dtype, band=band)["W0"]
    return W, W0


def _check(N, K, r, q, W, W0, dtype, what, oversample=10):
    l = B.probe_width(N, K, r, oversample)
    om = I.gaussian_probe("decompose", N + K + r, l, K) if r > 0 else np.zeros((0, K))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s, U, Vt = B.decompose(_dev(W, tdt), _dev(W0, tdt), r, torch.from_numpy(om).to(dev()), q=q)
    s, U, Vt = s.cpu().numpy(), U.cpu().numpy(), Vt.cpu().numpy()
    so, Uo, Vto, So = oracle.decompose_randomized(W, W0, r, om, q)
    assert np.max(np.abs(s - so)) <= TOL_S * np.max(np.abs(so)), f"{what}: s"
    if r == 0:
        return
    P, Po = U @ Vt, Uo @ Vto
    scale = np.max(np.abs(Po))
    err = np.max(np.abs(P - Po)) / (scale if scale > 0 else 1.0)
    assert err <= TOL_UV or (scale == 0 and np.max(np.abs(P)) == 0), f"{what}: U Vt rel err {err:.3e}"
    # validity of the factors: U's columns orthogonal with the singular values
    # as norms, Vt's rows orthonormal (rows of zero singular value are zero)
    nz = So[:r] > 1e-12 * So[0] if So[0] > 0 else np.zeros(r, bool)
    assert np.allclose(np.linalg.norm(U, axis=0)[nz], So[:r][nz], rtol=1e-9), what
    G = Vt[nz] @ Vt[nz].T
    assert np.allclose(G, np.eye(int(nz.sum())), atol=1e-9), what
    return err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 2, 3, 7])
def test_band_mean_bit_exact(L, dtype):
    """W0 = the mean of the band's layer weights, rounded once: the same bits
    as the oracle's float64 mean rounded to the storage type."""
    N, K = 130, 264
    Ws = [I.trained_weight("decompose", l, "k", K, N, dtype, band=0) for l in range(L)]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    got = B.band_mean([_dev(w, tdt) for w in Ws]).float().cpu().numpy().astype(np.float64)
    ref = oracle.band_means(Ws, 1)[0]
    ref = oracle.rne_bf16(ref) if dtype == "bf16" else oracle.rne_f32(ref)
    assert np.array_equal(got, ref)
    if L == 1:
        assert np.array_equal(got, Ws[0].astype(np.float64))      # one layer per band: its own weight


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lsq_scale_and_zero_rows(dtype):
    """r = 0: the scale only; rows of W0 that are zero get s = 1."""
    N, K = 77, 200
    W, W0 = _weights(N, K, 4, 1, dtype)
    W0 = W0.copy()
    W0[[3, 40]] = 0.0
    _check(N, K, 0, 0, W, W0, dtype, "r=0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    s, _, _ = B.decompose(_dev(W, tdt), _dev(W0, tdt), 0, None)
    assert float(s[3]) == 1.0 and float(s[40]) == 1.0


@pytest.mark.parametrize("N,K,r,q", [(300, 520, 8, 2), (520, 300, 8, 0), (600, 700, 16, 3), (333, 1048, 4, 1)])
def test_decompose_randomized(N, K, r, q):
    """min(N, K) > 256: the randomized branch, with and without subspace steps,
    tall and wide."""
    W, W0 = _weights(N, K, r, 2)
    _check(N, K, r, q, W, W0, "bf16", f"{N}x{K} r={r} q={q}")


@pytest.mark.parametrize("N,K,r", [(256, 256, 4), (200, 264, 6), (96, 1152, 8), (1024, 100, 10)])
def test_decompose_full_svd_rule(N, K, r):
    """min(N, K) <= 256: the pages' full SVD, here the same steps with a probe
    covering the matrix (l = min(N, K); 256 takes the kernels' paths with the
    l x l matrices in global memory)."""
    W, W0 = _weights(N, K, r, 3, "f32")
    _check(N, K, r, 1, W, W0, "f32", f"{N}x{K} r={r}")


def test_decompose_passthrough_and_rank_deficient():
    """W0 = W: s = 1 and a zero residual, so U Vt = 0; a residual of rank 3
    below r = 8: the probe's basis loses the missing directions (dropped
    columns) and U Vt is the residual itself."""
    N, K = 300, 400
    W, W0 = _weights(N, K, 4, 4, "f32")
    _check(N, K, 6, 2, W, W, "f32", "passthrough")
    rng = np.random.default_rng(5)
    R3 = (rng.standard_normal((N, 3)) @ rng.standard_normal((3, K)) * 1e-3).astype(np.float32)
    Wd = (W0.astype(np.float64) * 1.05 + R3).astype(np.float32)
    _check(N, K, 8, 1, Wd, W0, "f32", "rank 3")


@pytest.mark.parametrize("fam,r", [("q", 16), ("gate", 64), ("down", 64), ("k", 64)])
def test_decompose_gemma_shapes(fam, r):
    """Gemma-3-1B-shaped projections (bf16): q 1152 -> 1024 at rank 16, gate
    1152 -> 6912 and down 6912 -> 1152 at rank 64, and k 1152 -> 256 at rank
    64 (min(N, K) = 256: the full SVD, l = N, on the block eigensolver)."""
    K, N = I.GEMMA_1B[fam]
    W, W0 = _weights(N, K, r, 5, "bf16", family=fam)
    _check(N, K, r, 2, W, W0, "bf16", f"{fam} r={r}")


def test_decompose_band_end_to_end():
    """Two layers of one band: W0 = their band mean, then each layer's bundle;
    GPU (band mean, decompose) against the oracle (band mean, decomposition) on
    the scale and on the size of what the rank-r term leaves, which the
    randomized SVD brings within 1e-6 of the Eckart-Young optimum here."""
    N, K, r = 640, 576, 12
    Ws = [I.trained_weight("decompose", l, "o", K, N, "bf16", band=1, waves=6) for l in (0, 1)]
    W0d = B.band_mean([_dev(w, torch.bfloat16) for w in Ws])
    W0o = oracle.rne_bf16(oracle.band_means(Ws, 1)[0])
    l = B.probe_width(N, K, r)
    om = I.gaussian_probe("decompose", 77, l, K)
    for Wl in Ws:
        s, U, Vt = B.decompose(_dev(Wl, torch.bfloat16), W0d, r, torch.from_numpy(om).to(dev()), q=3)
        so, Uo, Vto, So = oracle.decompose_randomized(Wl, W0o, r, om, 3)
        s, U, Vt = s.cpu().numpy(), U.cpu().numpy(), Vt.cpu().numpy()
        assert rel_err(s, so) <= TOL_S
        R = Wl.astype(np.float64) - so[:, None] * W0o
        e_gpu = np.linalg.norm(R - U @ Vt)
        e_ora = np.linalg.norm(R - Uo @ Vto)
        opt = np.sqrt(np.sum(np.linalg.svd(R, compute_uv=False)[r:] ** 2))
        assert abs(e_gpu - e_ora) <= 1e-6 * e_ora
        assert e_gpu <= opt * (1 + 1e-6)


def test_decompose_leaves_recon_counters_zero():
    """The decomposition shares the default workspace with the recon calls:
    its scratch must not touch the reserved counter words that the prefill
    hand-off depends on (a dirty word would let waiters read t before it is
    written).  Decompose, then check the words and run a prefill with a
    rank-r hand-off on the same workspace."""
    N, K, r = 600, 700, 16
    W, W0 = _weights(N, K, r, 6)
    _check(N, K, r, 1, W, W0, "bf16", "before the recon call")
    ws = B.default_workspace()
    ws.check()
    M, Kr, Nr, rr = 200, 512, 160, 100
    bd = I.bundle("test", rr, "q", Kr, Nr, rr, "bf16", variant="s0")
    x = I.activations("test", rr, M, Kr, "bf16")
    y = B.recon_linear(up(x, "bf16"), bundle_up(bd, "bf16"))
    ws.check()
    assert rel_err(down(y), oracle.recon_linear(x, *bundle_np(bd))) <= 1e-2


def test_decompose_refusals():
    d = dev()
    W = torch.zeros((64, 128), dtype=torch.bfloat16, device=d)
    om = torch.zeros((300, 128), dtype=torch.float64, device=d)
    with pytest.raises(B.AQError) as e:                # l > min(N, K)
        B.decompose(W, W, 4, om[:100])
    assert e.value.status == B.AQ_ERR_SHAPE
    with pytest.raises(B.AQError) as e:                # l < r
        B.decompose(W, W, 8, om[:4])
    assert e.value.status == B.AQ_ERR_SHAPE


@pytest.mark.parametrize("N,K,r,oversample,jac,wgs", [
    (300, 520, 8, 10, 2, 1),      # l = 18 on the many-workgroup solver: one workgroup
    (300, 520, 8, 10, 2, 7),      # seven (rounds split unevenly)
    (300, 520, 8, 11, 2, 64),     # l = 19 (odd: a dummy index), the most workgroups
    (300, 520, 8, 11, 1, 0),      # l = 19 in LDS
    (95, 300, 5, 10, 0, 0),       # l = N = 95: Q = I, the largest odd l in LDS
    (95, 300, 5, 10, 2, 5),       # the same on the grid
    (97, 400, 6, 10, 0, 0),       # l = N = 97: the block solver by default (odd, padded to 128)
    (97, 400, 6, 10, 2, 3),       # the scalar grid solver on three workgroups
    (500, 128, 8, 10, 0, 0),      # l = K = 128: no subspace steps, the packed Cholesky at its limit
    (600, 150, 8, 10, 0, 0),      # l = K = 150: the Cholesky in global memory (block solver, 192)
    (150, 500, 12, 10, 2, 0),     # l = N = 150 on the scalar grid solver
    (256, 700, 16, 10, 0, 0),     # l = N = 256: the block solver at its largest (four sets of 64)
    (400, 600, 40, 10, 0, 0),     # l = 50: the 64-wide contraction tiles
    (400, 600, 40, 10, 3, 0),     # l = 50 on the block solver (one set: n padded to 64)
    (300, 520, 8, 11, 3, 0),      # l = 19 on the block solver
    (129, 400, 5, 10, 0, 0),      # l = N = 129: padded to 192 (63 zero rows), three sets
    (193, 400, 7, 10, 0, 0),      # l = N = 193: padded to 256
    (96, 300, 5, 10, 3, 0),       # l = N = 96 forced onto the block solver (padded to 128)
])
def test_decompose_eigensolvers(N, K, r, oversample, jac, wgs, force_plan):
    """The three Jacobi eigensolvers (one workgroup with G and V in LDS; the
    scalar one over many workgroups with a grid barrier per round; the block
    one, 64 x 64 subproblems in LDS and block updates between grid barriers)
    at odd and even l, several grid sizes, and both Cholesky kernels."""
    if jac:
        force_plan("JACOBI", jac)
    if wgs:
        force_plan("JACOBI_WGS", wgs)
    W, W0 = _weights(N, K, r, 7, "f32")
    _check(N, K, r, 2, W, W0, "f32", f"{N}x{K} r={r} p={oversample} jacobi={jac} wgs={wgs}", oversample)


@pytest.mark.parametrize("jac", [0, 2])
def test_decompose_grid_give_up_reported(jac, force_plan):
    """A grid barrier of the many-workgroup eigensolvers (block: the default
    at l = 200; scalar) that gives up (forced from the host: one more arrival
    awaited than will come, 64 polls): every workgroup exits, U and Vt are
    NaN, and the workspace check reports it (and clears it); the next call on
    that workspace is valid."""
    if jac:
        force_plan("JACOBI", jac)
    N, K, r = 200, 264, 6
    W, W0 = _weights(N, K, r, 8, "f32")
    Wd, W0d = _dev(W, torch.float32), _dev(W0, torch.float32)
    om = torch.zeros((N, K), dtype=torch.float64, device=dev())      # l = N: Q = I, omega unused
    ws = B.Workspace()
    force_plan("HANDOFF_SPIN", 64)
    force_plan("HANDOFF_UNREACHABLE", 1)
    s, U, Vt = B.decompose(Wd, W0d, r, om, q=1, workspace=ws)
    assert torch.isnan(U).all() and torch.isnan(Vt).all()
    with pytest.raises(B.AQError) as e:
        ws.check()
    assert e.value.status == B.AQ_ERR_HANDOFF, e.value
    B.aq_debug_reset_plan()
    if jac:
        force_plan("JACOBI", jac)
    s, U, Vt = B.decompose(Wd, W0d, r, om, q=1, workspace=ws)
    ws.check()
    so, Uo, Vto, _ = oracle.decompose_randomized(W, W0, r, np.zeros((N, K)), 1)
    Po = Uo @ Vto
    assert np.max(np.abs(U.cpu().numpy() @ Vt.cpu().numpy() - Po)) <= TOL_UV * np.max(np.abs(Po))
