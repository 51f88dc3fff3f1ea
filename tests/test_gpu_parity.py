"""GPU parity: the HIP library (through the C ABI) against the CPU fp64 oracle on
the same seeded inputs.  Small shapes span several tiles and ragged tails; the
workload shapes are checked in full (decode) or on sampled tokens and output
columns (prefill, large decoder)."""

import numpy as np
import pytest
import torch

import oracle
from rank_shared_block_amd import binding as B
from rank_shared_block_amd import inputs as I
from helpers import (assert_parity, bundle_np, bundle_up, dev, down, rel_err, sub_bundle, up)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    d = dev()
    B.lib()
    assert len(B.hip_runtimes_mapped()) == 1, B.hip_runtimes_mapped()
    torch.cuda.synchronize(d)
    yield


def _single(M, K, N, r, dtype, variant="normal", layer=0, tag=0):
    bd = I.bundle("test", layer, "q", K, N, r, dtype, variant=variant)
    x = I.activations("test", tag, M, K, dtype)
    return bd, x


# ------------------------------------------------------------- fp32 (C1)

@pytest.mark.parametrize("variant", ["normal", "r0", "passthrough", "s0"])
def test_single_projection_f32(variant):
    bd = I.bundle("single_f32", 0, "q", 256, 256, 4, "f32", variant=variant)
    x = I.activations("single_f32", 0, 8, 256, "f32")
    y = B.recon_linear(up(x, "f32"), bundle_up(bd, "f32"))
    ref = oracle.recon_linear(x, *bundle_np(bd))
    assert_parity(down(y), ref, "f32", variant)
    w = B.materialize(bundle_up(bd, "f32"))
    wref = oracle.materialize(*bundle_np(bd))
    if variant in ("r0", "passthrough"):
        assert np.array_equal(down(w), oracle.rne_f32(wref))      # one rounding: bit-exact
    else:
        assert_parity(down(w), wref, "f32", "materialize " + variant)


@pytest.mark.parametrize("M", [1, 5, 17, 40])
def test_f32_ragged(M):
    bd, x = _single(M, 132, 70, 9, "f32")
    y = B.recon_linear(up(x, "f32"), bundle_up(bd, "f32"))
    assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bd)), "f32")


# ------------------------------------------------------------- bf16 recon, small

@pytest.mark.parametrize("M", [1, 3, 5, 16, 17, 33, 64, 65, 130, 300])
@pytest.mark.parametrize("variant", ["normal", "s0"])
def test_bf16_batch_sizes(M, variant):
    """Every batch bucket (streaming 16/32/64-token kernels, tiled MFMA beyond)
    with a ragged N (200), a K that is not a tile multiple (1048) and r = 24."""
    bd, x = _single(M, 1048, 200, 24, "bf16", variant=variant, tag=M)
    y = B.recon_linear(up(x, "bf16"), bundle_up(bd, "bf16"))
    assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bd)), "bf16", f"M={M} {variant}")


@pytest.mark.parametrize("r", [0, 5, 16, 40, 100, 256])
@pytest.mark.parametrize("M", [4, 200])
def test_bf16_ranks(r, M):
    bd, x = _single(M, 512, 160, r, "bf16", variant="s0" if r else "normal", layer=r, tag=r)
    y = B.recon_linear(up(x, "bf16"), bundle_up(bd, "bf16"))
    assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bd)), "bf16", f"r={r} M={M}")


@pytest.mark.parametrize("M", [16, 300])
def test_bf16_rank0_and_passthrough_agree(M, force_plan):
    """Passthrough (s = 1, U = Vt = 0, W0 = the layer's own weight) and r = 0
    with s = 1 give the same bits (the W0 contraction's summation order does not
    depend on r, and the rank term adds exact zeros), at a decode batch (the
    streaming kernel, its fused mode forced for both so that the K split is the
    same) and at a prefill batch (the tiled kernel); both are within tolerance
    of x W^T ("How attnquant works", section "The passthrough operating
    point")."""
    K, N = 1024, 300
    if M <= 64:
        force_plan("DECODE_SPLIT", 0)
    bd = I.bundle("test", 7, "o", K, N, 16, "bf16", variant="passthrough")
    x = up(I.activations("test", 7 + M, M, K, "bf16"), "bf16")
    W0, s, U, Vt = bundle_up(bd, "bf16")
    y_pt = B.recon_linear(x, (W0, s, U, Vt))
    y_r0 = B.recon_linear(x, (W0, s, None, None))
    torch.cuda.synchronize()
    assert torch.equal(y_pt, y_r0), f"M={M}: passthrough and r = 0 differ"
    ref = down(x) @ bd["W0"].astype(np.float64).T
    assert_parity(down(y_pt), ref, "bf16", "passthrough")
    assert_parity(down(y_r0), ref, "bf16", "r0")


@pytest.mark.parametrize("M", [1, 16, 40, 300])
def test_fused_qkv_small(M):
    K = 264
    shapes = [(96, 8), (40, 16), (24, 0)]
    bds = [I.bundle("test", 1, f, K, n, r, "bf16") for f, (n, r) in zip(("q", "k", "v"), shapes)]
    x = I.activations("test", 100 + M, M, K, "bf16")
    y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    ref = oracle.recon_fused(x, [bundle_np(b) for b in bds])
    assert y.shape == (M, 160)
    assert_parity(down(y), ref, "bf16", f"qkv M={M}")
    # block-diagonal: each block's columns equal the single-projection call
    col = 0
    for b in bds:
        n = b["W0"].shape[0]
        assert_parity(down(y)[:, col:col + n], oracle.recon_linear(x, *bundle_np(b)), "bf16")
        col += n


# The streaming kernel meets the rank-r term either inside each workgroup (fused)
# or with Vt rows as tiles of their own plus a combine kernel (split, with K
# split over S workgroups).  The host picks one per dispatch; both are forced
# here, over tile heights (NG 16-row groups) and split counts.
_DECODE_MODES = [("0", None, None), ("1", None, None), ("1", 1, 1), ("1", 2, 3), ("1", 3, 7),
                 ("1", 4, 2), ("1", 6, 5)]


@pytest.mark.parametrize("M", [1, 7, 20, 40, 64])
@pytest.mark.parametrize("split,ng,S", _DECODE_MODES)
def test_decode_modes_qkv(M, split, ng, S, force_plan):
    force_plan("DECODE_SPLIT", int(split))
    if ng is not None:
        force_plan("DECODE_NG", ng)
    if S is not None:
        force_plan("DECODE_S", S)
    K = 1048
    shapes = [(200, 8), (40, 16), (24, 0)]
    bds = [I.bundle("test", 3, f, K, n, r, "bf16", variant="s0" if f == "q" else "normal")
           for f, (n, r) in zip(("q", "k", "v"), shapes)]
    x = I.activations("test", 400 + M, M, K, "bf16")
    y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16",
                  f"M={M} split={split} NG={ng} S={S}")


@pytest.mark.parametrize("M", [1, 16, 20, 64])
@pytest.mark.parametrize("rows", [5, 17, 27, 54, 64, 80])
def test_decode_fused_rows(M, rows, force_plan):
    """Fused tiles of any row count (not a multiple of 16; the last tile of each
    block shorter still), over a fused gate/up pair with ragged N and K.  Row
    counts that no compiled tile of the batch bucket holds fall back to the plan."""
    force_plan("DECODE_SPLIT", 0)
    force_plan("DECODE_ROWS", rows)
    K = 1048
    bds = [I.bundle("test", 4, f, K, 333, 16, "bf16", variant="s0" if f == "gate" else "normal")
           for f in ("gate", "up")]
    x = I.activations("test", 600 + M, M, K, "bf16")
    y = B.recon_gateup(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16", f"M={M} rows={rows}")


@pytest.mark.parametrize("M", [1, 16, 33, 64])
@pytest.mark.parametrize("r", [49, 100, 256])
def test_decode_high_rank_split(M, r):
    """Ranks that no fused tile holds go to split mode (Vt rows as their own tiles)."""
    bd, x = _single(M, 2048, 136, r, "bf16", variant="s0", layer=r, tag=500 + M)
    y = B.recon_linear(up(x, "bf16"), bundle_up(bd, "bf16"))
    assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bd)), "bf16", f"r={r} M={M}")


@pytest.mark.parametrize("M,S", [(33, 1), (33, 3), (64, 2), (9, 1)])
@pytest.mark.parametrize("ranks", [(32, 32), (48, 0), (36, 100)], ids=str)
def test_decode_combine_token_groups(M, S, ranks, force_plan):
    """Split mode on a wide gate/up pair (the combine launches more than 2048
    workgroups of one token each), K in one or more ranges, token counts off
    the 16-token groups of the streaming kernel (33, 9); U rows of up to 32
    ranks requested before the barrier, longer 16-byte aligned rows (48), rows
    that are not 16-byte aligned (36, 100), a block without rank."""
    force_plan("DECODE_SPLIT", 1)
    force_plan("DECODE_S", S)
    K = 768
    bds = [I.bundle("test", 10, f, K, 9000, r, "bf16", variant="s0" if f == "up" else "normal")
           for f, r in zip(("gate", "up"), ranks)]
    x = I.activations("test", 1200 + M + S, M, K, "bf16")
    y = B.recon_gateup(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16", f"M={M} S={S} r={ranks}")


# The tiled kernel: every compiled tile shape (BM x BN output, BK-wide K slices
# through NST LDS stages), forced K splits of the main pass and of the rank-r
# pass, on ragged M, N and K (K = 1048 leaves a partial last K slice; N = 200,
# 40, 24 leave partial column tiles; r = 8, 16, 0).
_PREFILL_MODES = [None, (256, 256, 32, 4, 1, None), (256, 256, 64, 2, 1, None), (256, 128, 64, 3, 1, 1),
                  (128, 256, 64, 3, 1, 3), (128, 128, 64, 2, 1, None), (128, 128, 64, 4, 2, 5),
                  (256, 256, 32, 4, 3, 2), (256, 256, 64, 2, 3, 2), (256, 128, 64, 3, 2, None),
                  (256, 128, 32, 3, 1, None), (128, 256, 32, 3, 2, 1), (128, 128, 32, 4, 1, None),
                  (64, 64, 64, 4, 1, None), (64, 128, 64, 4, 2, None), (128, 64, 64, 4, 1, 3),
                  (256, 256, 32, 4, 1, None, 8), (256, 256, 64, 2, 1, None, 8), (256, 256, 32, 4, 2, 2, 8),
                  (128, 96, 64, 4, 1, None), (128, 96, 64, 4, 3, None), (128, 96, 64, 4, 1, 2)]


@pytest.mark.parametrize("M", [65, 300, 513])
@pytest.mark.parametrize("mode", _PREFILL_MODES, ids=str)
def test_prefill_modes_qkv(M, mode, force_plan):
    if mode is not None:
        bm, bn, bk, nst, S, tS = mode[:6]
        nw = mode[6] if len(mode) > 6 else 4
        for k, v in (("BM", bm), ("BN", bn), ("BK", bk), ("NST", nst), ("S", S), ("W", nw)):
            force_plan(f"PREFILL_{k}", v)
        if tS is not None:
            force_plan("TPASS_S", tS)
    K = 1048
    shapes = [(200, 8), (40, 16), (24, 0)]
    bds = [I.bundle("test", 4, f, K, n, r, "bf16", variant="s0" if f == "k" else "normal")
           for f, (n, r) in zip(("q", "k", "v"), shapes)]
    x = I.activations("test", 600 + M, M, K, "bf16")
    y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16", f"M={M} mode={mode}")


@pytest.mark.parametrize("M", [65, 1000])
@pytest.mark.parametrize("K", [40, 1048, 6912])
def test_rank_pass_shapes(M, K):
    """The rank-r pass over short and long K, ranks of 1, 2 and 4 chunks of 64."""
    shapes = [(64, 130), (48, 64), (40, 250)]
    bds = [I.bundle("test", 9, f, K, n, r, "bf16", variant="s0") for f, (n, r) in zip(("q", "k", "v"), shapes)]
    x = I.activations("test", 800 + M + K, M, K, "bf16")
    y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16", f"M={M} K={K}")


@pytest.mark.parametrize("M", [80, 600])
@pytest.mark.parametrize("r", [36, 64, 100, 256])
@pytest.mark.parametrize("tile", [(256, 256, 32, 4), (256, 256, 64, 2), (256, 128, 64, 3), (128, 256, 32, 3),
                                  (256, 256, 32, 4, 8), (256, 256, 64, 2, 8)], ids=str)
def test_prefill_high_rank(M, r, tile, force_plan):
    """Rank-r epilogues over one or several rank chunks (some riding on the tail
    of the K ring, the rest read from global memory), with U rows that are
    16-byte aligned (r % 8 == 0) or not (r = 36, 100); four- and eight-wave
    workgroups."""
    for k, v in zip(("BM", "BN", "BK", "NST", "W"), tuple(tile) + ((4,) if len(tile) == 4 else ())):
        force_plan(f"PREFILL_{k}", v)
    bd, x = _single(M, 512, 520, r, "bf16", variant="s0", layer=r, tag=700 + M)
    y = B.recon_linear(up(x, "bf16"), bundle_up(bd, "bf16"))
    assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bd)), "bf16", f"r={r} M={M}")


@pytest.mark.parametrize("M", [300, 700])
@pytest.mark.parametrize("K", [1048, 3000])
@pytest.mark.parametrize("S", [1, 3])
@pytest.mark.parametrize("tile", [(128, 128, 64, 4, 4), (128, 96, 64, 4, 4), (256, 128, 32, 3, 4), (256, 256, 32, 4, 8)], ids=str)
def test_prefill_rank_pass_in_main_launch(M, K, S, tile, force_plan):
    """The rank-r pass run by the first workgroups of the main-pass launch
    (these shapes leave free slots in the last round), with K short and long
    (unsplit), or the main pass K-split in three with one t per K range; U rows
    16-byte aligned (r = 16) and not (r = 36, read per round from global
    memory), a block without rank; the arrival counters are back at zero after
    every call."""
    for k, v in zip(("BM", "BN", "BK", "NST", "W", "S"), tuple(tile) + (S,)):
        force_plan(f"PREFILL_{k}", v)
    shapes = [(300, 16), (200, 36), (72, 0)]
    bds = [I.bundle("test", 6, f, K, n, r, "bf16", variant="normal") for f, (n, r) in zip(("q", "k", "v"), shapes)]
    x = I.activations("test", 950 + M + K, M, K, "bf16")
    ref = oracle.recon_fused(x, [bundle_np(b) for b in bds])
    for rep in range(2):
        y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
        assert_parity(down(y), ref, "bf16", f"M={M} K={K} tile={tile} rep={rep}")
        torch.cuda.synchronize()
        counters = B.default_workspace()._buf[torch.device(dev()).index][:576].cpu()
        assert int(counters.sum()) == 0, counters


@pytest.mark.parametrize("M", [130, 300])
@pytest.mark.parametrize("K", [200, 1048])
@pytest.mark.parametrize("parts", [2, 3, 4])
def test_prefill_rank_pass_in_parts(M, K, parts, force_plan):
    """Main tiles of 64 x 64 with the rank-r pass in the same launch, its K split
    into parts that are kept apart and summed by the main tiles' epilogue: two
    or three parts ride the LDS ring, a fourth goes the per-round path; U rows
    aligned (r = 16) and not (r = 36); K = 200 allows two parts of >= 128 K
    values only.  The workspace size shows that the plan keeps the parts."""
    for k, v in zip(("BM", "BN", "BK", "NST", "W"), (64, 64, 64, 4, 4)):
        force_plan(f"PREFILL_{k}", v)
    force_plan("TPASS_PARTS", parts)
    force_plan("PREFILL_SELF", 0)
    shapes = [(300, 16), (200, 36), (72, 0)]
    bds = [I.bundle("test", 7, f, K, n, r, "bf16", variant="normal") for f, (n, r) in zip(("q", "k", "v"), shapes)]
    nparts = min(parts, (K + 127) // 128)
    ldt = 16 + 48
    fake = [B.aq_proj(n, r, 256, 256, 256, 256) for n, r in shapes]
    want = 65536 + (M * ldt * 2 * nparts + 255) // 256 * 256
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, M, K, fake, 3) == want
    x = I.activations("test", 970 + M + K, M, K, "bf16")
    ref = oracle.recon_fused(x, [bundle_np(b) for b in bds])
    for rep in range(2):
        y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
        assert_parity(down(y), ref, "bf16", f"M={M} K={K} parts={parts} rep={rep}")
        torch.cuda.synchronize()
        counters = B.default_workspace()._buf[torch.device(dev()).index][:576].cpu()
        assert int(counters.sum()) == 0, counters


def test_prefill_handoff_give_up_is_reported(force_plan):
    """The bounded wait of the main tiles for the rank-r workgroups of their
    launch: with the awaited count forced one above what arrives and the wait
    bounded to 64 polls, every kernel still exits, the flag is set and
    aq_workspace_check reports it (and clears the workspace); the next call,
    with the plan back to normal, is correct and leaves the workspace clean."""
    M, K = 300, 1048
    shapes = [(300, 16), (200, 36), (72, 0)]
    bds = [I.bundle("test", 6, f, K, n, r, "bf16", variant="normal") for f, (n, r) in zip(("q", "k", "v"), shapes)]
    x = I.activations("test", 960, M, K, "bf16")
    ref = oracle.recon_fused(x, [bundle_np(b) for b in bds])
    ws = B.Workspace()
    for k, v in zip(("BM", "BN", "BK", "NST", "W"), (128, 128, 64, 4, 4)):
        force_plan(f"PREFILL_{k}", v)
    force_plan("HANDOFF_SPIN", 64)
    force_plan("HANDOFF_UNREACHABLE", 1)
    B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds], workspace=ws)
    with pytest.raises(B.AQError) as e:
        ws.check()
    assert e.value.status == B.AQ_ERR_HANDOFF, e.value
    assert int(ws._buf[torch.device(dev()).index][:576].cpu().sum()) == 0
    B.aq_debug_reset_plan()
    for k, v in zip(("BM", "BN", "BK", "NST", "W"), (128, 128, 64, 4, 4)):
        force_plan(f"PREFILL_{k}", v)
    y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds], workspace=ws)
    assert_parity(down(y), ref, "bf16", "after the reported give-up")
    ws.check()


@pytest.mark.parametrize("M", [65, 130, 300])
@pytest.mark.parametrize("K", [200, 1048, 2000])
@pytest.mark.parametrize("tile", [(64, 64, 64, 4), (128, 128, 32, 4), (128, 128, 64, 3), (128, 96, 64, 4),
                                  (128, 96, 64, 3)])
def test_prefill_own_t(M, K, tile, force_plan):
    """Main tiles that compute their own rows of t (Vt rows as more B rows of
    every stage, t rounded to bf16 in LDS, one or two rank chunks; K <= 2048):
    r = 64, r = 16, r = 36 (U rows not 16-byte aligned: the per-round path
    with t from LDS), a block without rank; nothing in the workspace.  Two or
    four wave rows (128 x 96: one wave column, two t blocks per wave)."""
    for k, v in zip(("BM", "BN", "BK", "NST", "W"), tuple(tile) + (4,)):
        force_plan(f"PREFILL_{k}", v)
    shapes = [(300, 64), (200, 16), (136, 36), (72, 0)]
    bds = [I.bundle("test", 8, f, K, n, r, "bf16", variant="normal") for f, (n, r) in zip(("q", "k", "v", "o"), shapes)]
    fake = [B.aq_proj(n, r, 256, 256, 256, 256) for n, r in shapes[:3]]
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, M, K, fake, 3) == 0
    x = I.activations("test", 990 + M + K, M, K, "bf16")
    for sel in ((0, 1, 2), (1, 2, 3)):
        sub = [bds[i] for i in sel]
        y = B.recon_qkv(up(x, "bf16"), [bundle_up(b, "bf16") for b in sub])
        assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in sub]), "bf16", f"M={M} K={K} {sel}")
    y = B.recon_linear(up(x, "bf16"), bundle_up(bds[0], "bf16"))
    assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bds[0])), "bf16", f"single M={M} K={K}")


@pytest.mark.parametrize("M", [1, 16, 33, 130])
def test_fused_gateup_small(M):
    K = 384
    bds = [I.bundle("test", 2, f, K, 272, 24, "bf16", variant="s0") for f in ("gate", "up")]
    x = I.activations("test", 200 + M, M, K, "bf16")
    y = B.recon_gateup(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16")


@pytest.mark.parametrize("M", [3, 100])
def test_strided_x_and_y(M):
    """ldx > K and ldy > N: only the addressed columns are written."""
    K, N = 256, 48
    bd, x = _single(M, K, N, 8, "bf16", tag=300 + M)
    xb = torch.zeros((M, K + 24), dtype=torch.bfloat16, device=dev())
    xb[:, :K] = up(x, "bf16")
    yb = torch.full((M, N + 40), 7.0, dtype=torch.bfloat16, device=dev())
    B.recon_linear(xb[:, :K], bundle_up(bd, "bf16"), y=yb[:, 8:8 + N])
    got = down(yb)
    assert np.all(got[:, :8] == 7.0) and np.all(got[:, 8 + N:] == 7.0)
    assert_parity(got[:, 8:8 + N], oracle.recon_linear(x, *bundle_np(bd)), "bf16")


def test_empty_batch_is_noop():
    bd, _ = _single(1, 128, 32, 4, "bf16")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device=dev())
    y = B.recon_linear(x, bundle_up(bd, "bf16"))
    assert y.shape == (0, 32)


def test_deterministic_and_workspace_reuse():
    """Repeated calls give identical bits; calls of different shapes share one
    workspace (its split-K counters reset themselves)."""
    K = 6912
    bd = I.bundle("test", 3, "down", K, 1152, 16, "bf16")
    W = bundle_up(bd, "bf16")
    outs = []
    for M in (1, 16, 1, 16, 7):
        x = up(I.activations("test", 400 + M, M, K, "bf16"), "bf16")
        outs.append((M, B.recon_linear(x, W)))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][1], outs[2][1]) and torch.equal(outs[1][1], outs[3][1])
    for M, y in outs:
        x = I.activations("test", 400 + M, M, K, "bf16")
        assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bd)), "bf16", f"M={M}")


# ------------------------------------------------------------- workload shapes

def _layer_dispatches(shapes, layer_bd):
    for name, fams in I.LAYER_DISPATCHES:
        K = shapes[fams[0]][0]
        yield name, fams, K, [layer_bd[f] for f in fams]


def _run_dispatch(name, x_dev, bds_dev):
    if name == "qkv":
        return B.recon_qkv(x_dev, bds_dev)
    if name == "gateup":
        return B.recon_gateup(x_dev, bds_dev)
    return B.recon_linear(x_dev, bds_dev[0])


@pytest.mark.parametrize("M", [1, 4, 16])
def test_gemma_decode_layer_full(M):
    lb = I.layer_bundles("gemma_decode", I.GEMMA_1B, layers=1, r=16, dtype="bf16")[0]
    for name, fams, K, bds in _layer_dispatches(I.GEMMA_1B, lb):
        x = I.activations("gemma_decode", 10 * M + len(name), M, K, "bf16")
        y = _run_dispatch(name, up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
        ref = oracle.recon_fused(x, [bundle_np(b) for b in bds])
        assert_parity(down(y), ref, "bf16", f"gemma decode {name} M={M}")


@pytest.mark.parametrize("M", [512, 2048])
def test_gemma_prefill_layer_sampled(M):
    lb = I.layer_bundles("gemma_prefill", I.GEMMA_1B, layers=1, r=64, dtype="bf16")[0]
    rng = np.random.default_rng(M)
    rows = np.sort(rng.choice(M, 48, replace=False))
    for name, fams, K, bds in _layer_dispatches(I.GEMMA_1B, lb):
        x = I.activations("gemma_prefill", M + len(name), M, K, "bf16")
        y = down(_run_dispatch(name, up(x, "bf16"), [bundle_up(b, "bf16") for b in bds]))
        ref = oracle.recon_fused(x[rows], [bundle_np(b) for b in bds])
        assert_parity(y[rows], ref, "bf16", f"gemma prefill {name} M={M}")
        assert np.all(np.isfinite(y))


def _strided_sample(rng, n, stride):
    """One index in every `stride`-wide window of range(n) (random offset per
    window): every tile of that width or wider is hit."""
    return np.array([w + rng.integers(0, min(stride, n - w)) for w in range(0, n, stride)])


@pytest.mark.parametrize("M", [1, 32, 512])
def test_large_decoder_banded_sampled(M):
    """Two layers of one W0 band (per-layer s, U, Vt), every dispatch: one
    output column in every 64-column window of every block (so every output
    tile and, with it, every tile of t it reads is compared) on one token in
    every 32-token window (every M tile)."""
    lbs = I.layer_bundles("large_decoder", I.LARGE_DECODER, layers=2, r=32, dtype="bf16",
                          num_bands=1)
    rng = np.random.default_rng(1000 + M)
    rows = np.unique(_strided_sample(rng, M, 32))
    for layer in (0, 1):
        for name, fams, K, bds in _layer_dispatches(I.LARGE_DECODER, lbs[layer]):
            x = I.activations("large_decoder", 7 * M + 3 * layer + len(name), M, K, "bf16")
            y = down(_run_dispatch(name, up(x, "bf16"), [bundle_up(b, "bf16") for b in bds]))
            col0, cols_all, refs = 0, [], []
            for b in bds:
                n = b["W0"].shape[0]
                cols = _strided_sample(rng, n, 64)
                refs.append(oracle.recon_linear(x[rows], *sub_bundle(b, cols)))
                cols_all.append(col0 + cols)
                col0 += n
            got = y[np.ix_(rows, np.concatenate(cols_all))]
            assert_parity(got, np.concatenate(refs, axis=1), "bf16", f"large {name} L{layer} M={M}")
            assert np.all(np.isfinite(y))
        torch.cuda.empty_cache()


# ------------------------------------------------------------- materialise

@pytest.mark.parametrize("N,K,r", [(70, 136, 0), (70, 136, 7), (130, 1048, 16), (200, 520, 64),
                                   (64, 256, 100), (33, 64, 256)])
def test_materialize_bf16(N, K, r):
    bd = I.bundle("test", 5, "up", K, N, r, "bf16")
    w = B.materialize(bundle_up(bd, "bf16"))
    ref = oracle.materialize(*bundle_np(bd))
    if r == 0:
        assert np.array_equal(down(w), oracle.rne_bf16(ref))
    else:
        assert_parity(down(w), ref, "bf16", f"materialize N={N} K={K} r={r}")


def test_materialize_passthrough_bit_exact_and_strided():
    N, K = 96, 264
    bd = I.bundle("test", 6, "gate", K, N, 16, "bf16", variant="passthrough")
    stacked = torch.full((N + 10, K + 40), -3.0, dtype=torch.bfloat16, device=dev())
    B.materialize(bundle_up(bd, "bf16"), out=stacked[5:5 + N, :])
    got = down(stacked)
    assert np.array_equal(got[5:5 + N, :K], bd["W0"].astype(np.float64))
    assert np.all(got[5:5 + N, K:] == -3.0) and np.all(got[:5] == -3.0) and np.all(got[5 + N:] == -3.0)


@pytest.mark.parametrize("fam", ["q", "gate", "down"])
def test_materialize_gemma_r64(fam):
    K, N = I.GEMMA_1B[fam]
    bd = I.bundle("materialize_fp4", 0, fam, K, N, 64, "bf16")
    w = B.materialize(bundle_up(bd, "bf16"))
    assert_parity(down(w), oracle.materialize(*bundle_np(bd)), "bf16", f"materialize {fam}")


# ------------------------------------------------------------- FP4 pack

def _weff_seeded(bd):
    """A bundle's effective weight from the oracle, rounded once to bf16: a
    W_eff-shaped pack input that does not come from the HIP path."""
    return oracle.rne_bf16(oracle.materialize(*bundle_np(bd)))


def _fp4_check(w_dev):
    p, s, g = B.quant_fp4_block16(w_dev)
    ep, es, eg = oracle.fp4_pack(down(w_dev))
    assert float(g.cpu()[0]) == eg
    assert np.array_equal(s.cpu().numpy(), es)
    assert np.array_equal(p.cpu().numpy(), ep)


@pytest.mark.parametrize("N,K", [(1, 16), (37, 48), (130, 1056)])
def test_fp4_small(N, K):
    bd = I.bundle("test", 8, "v", K, N, 8, "bf16")
    _fp4_check(up(_weff_seeded(bd), "bf16"))


def test_fp4_edge_blocks():
    """All-zero rows and blocks, blocks far below the global max (subnormal and
    zero E4M3 scales), exact E2M1 midpoints, negative zeros."""
    rng = np.random.default_rng(9)
    W = rng.standard_normal((8, 64)).astype(np.float32)
    W[1] = 0.0
    W[2, :16] *= 1e-6
    W[3, 16:32] *= 1e-12
    W[4, :16] = -0.0
    W[5] = 0.0
    W[5, 0] = 10.5                      # this row: exact grid, ties at D = 1.75
    W[5, 1:8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 1.75
    W[0, 0] = 40.0                      # global max
    w = torch.from_numpy(W).to(torch.bfloat16).to(dev())
    _fp4_check(w)
    z = torch.zeros((4, 32), dtype=torch.bfloat16, device=dev())
    p, s, g = B.quant_fp4_block16(z)
    assert float(g.cpu()[0]) == 1.0 and not p.any() and not s.any()


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_fp4_near_midpoints(seed):
    """Values at and next to the E2M1 decision points m_i * D of their block,
    with D of full fp32 precision (g = A / 2688 for an A of many bits), so that
    m_i * D is not a float and the float-side tie decisions are exercised."""
    rng = np.random.default_rng(100 + seed)
    N, K = 48, 256
    A = float(torch.tensor(97.3 + seed, dtype=torch.bfloat16))
    g = oracle.fp4.global_scale(A)
    W = np.zeros((N, K))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for n in range(N):
        for b in range(K // 16):
            bmax = float(torch.tensor(rng.uniform(0.05, A), dtype=torch.bfloat16))
            sf = oracle.fp4.e4m3fn_encode_rne_sat(np.array([bmax / (6.0 * g)]))
            D = float(np.float32(g * oracle.fp4.e4m3fn_decode(sf)[0]))
            v = mids[rng.integers(0, 7, 15)] * D * (1.0 + rng.choice([-1, 0, 1], 15) * 2.0 ** -9)
            v = np.minimum(v, bmax)
            blk = np.concatenate([[bmax], v * rng.choice([-1.0, 1.0], 15)])
            W[n, 16 * b:16 * b + 16] = rng.permutation(blk)
    W[0, 0] = A
    w = torch.from_numpy(W).to(torch.bfloat16).to(dev())
    _fp4_check(w)


@pytest.mark.parametrize("fam", ["k", "down"])
def test_fp4_gemma_full(fam):
    K, N = I.GEMMA_1B[fam]
    bd = I.bundle("materialize_fp4", 1, fam, K, N, 64, "bf16")
    _fp4_check(up(_weff_seeded(bd), "bf16"))


def test_fp4_strided_source():
    N, K = 40, 96
    bd = I.bundle("test", 9, "o", K, N, 4, "bf16")
    big = torch.zeros((N, K + 32), dtype=torch.bfloat16, device=dev())
    wn = _weff_seeded(bd)
    big[:, :K] = up(wn, "bf16")
    p, s, g = B.quant_fp4_block16(big[:, :K])
    ep, es, eg = oracle.fp4_pack(wn)
    assert np.array_equal(p.cpu().numpy(), ep) and np.array_equal(s.cpu().numpy(), es)


# ------------------------------------------------------------- HIP graph capture

def test_graph_capture_replays_match_eager():
    """Decode (split-K counters in the workspace) and prefill (t buffer) calls
    captured in one graph: every replay, with eager work and synchronisations in
    between, reproduces the eager result bit for bit."""
    d = dev()
    bd_dec = I.bundle("test", 11, "down", 6912, 1152, 16, "bf16")
    bd_pf = I.bundle("test", 12, "q", 1152, 1024, 64, "bf16")
    Wd, Wp = bundle_up(bd_dec, "bf16"), bundle_up(bd_pf, "bf16")
    xd = up(I.activations("test", 500, 16, 6912, "bf16"), "bf16")
    xp = up(I.activations("test", 501, 300, 1152, "bf16"), "bf16")
    ws = B.Workspace()
    yd = B.recon_linear(xd, Wd, workspace=ws)
    yp = B.recon_linear(xp, Wp, workspace=ws)
    torch.cuda.synchronize()
    eager_d, eager_p = yd.clone(), yp.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.recon_linear(xd, Wd, y=yd, workspace=ws)
        B.recon_linear(xp, Wp, y=yp, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.recon_linear(xd, Wd, y=yd, workspace=ws)
        B.recon_linear(xp, Wp, y=yp, workspace=ws)
    for rep in range(4):
        yd.zero_()
        yp.zero_()
        B.recon_linear(xd[:3], Wd, workspace=ws)          # eager work on the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(yd, eager_d), f"decode replay {rep}"
        assert torch.equal(yp, eager_p), f"prefill replay {rep}"
    assert_parity(down(eager_d), oracle.recon_linear(I.activations("test", 500, 16, 6912, "bf16"),
                                                    *bundle_np(bd_dec)), "bf16")


def test_workspace_shared_across_call_kinds():
    """Split-K decode, prefill (rank-r scratch) and FP4 pack (partial maxima) on one
    workspace: the scratch of one never disturbs the counters of another."""
    ws = B.Workspace()
    bd = I.bundle("test", 13, "down", 6912, 1152, 16, "bf16")
    W = bundle_up(bd, "bf16")
    for M in (16, 300, 2, 129, 16):
        x = I.activations("test", 600 + M, M, 6912, "bf16")
        y = B.recon_linear(up(x, "bf16"), W, workspace=ws)
        assert_parity(down(y), oracle.recon_linear(x, *bundle_np(bd)), "bf16", f"M={M}")
        wn = _weff_seeded(bd)
        p, s, g = B.quant_fp4_block16(up(wn, "bf16"), workspace=ws)
        ep, es, eg = oracle.fp4_pack(wn)
        assert np.array_equal(p.cpu().numpy(), ep) and float(g.cpu()[0]) == eg


# ------------------------------------------------------------- FP4 decode GEMV

def _fp4_weight(N, K, seed):
    """A seeded bf16 weight (rows of different scales, so block steps vary) and
    its oracle pack."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * K ** -0.5 * np.exp2(rng.uniform(-2, 2, (N, 1)))
    Wb = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16)
    return Wb, oracle.fp4_pack(Wb.double().numpy())


def _assert_fp4_parity(got, x, p, s, g, what):
    """The spec bf16 tolerance, and elementwise the bound this arithmetic
    allows: each dequantised weight rounded once to bf16 (relative 2^-8 after an
    fp32 product, 2^-24; bf16's unit roundoff is 2^-8), exact bf16 x bf16
    products, fp32 sums of K terms (at most K 2^-24 of the sum of magnitudes),
    one bf16 rounding of the output.  (The kernel for up to four tokens skips
    the per-weight rounding; the bound covers both.)"""
    ref = oracle.fp4_linear(x, p, s, g)
    assert rel_err(got, ref) <= 1e-2, what
    absref = np.abs(np.asarray(x, dtype=np.float64)) @ np.abs(oracle.fp4_unpack(p, s, g)).T
    K = x.shape[1]
    bound = 2.0 ** -8 * np.abs(ref) + (2.0 ** -8 + 2.0 ** -23 + K * 2.0 ** -24) * absref * 1.01
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond the derived bound"


@pytest.mark.parametrize("M", [1, 3, 4, 16])
@pytest.mark.parametrize("N,K", [(300, 1152), (72, 96), (1152, 6912), (200, 2016), (4100, 1024), (50, 64)])
def test_fp4_linear(M, N, K):
    """FP4 GEMV against the oracle's product with the dequantised weight, from
    the oracle's pack: short K with a ragged tail step (96), long K split over
    workgroups with the fold (6912, 2016), wide N with 64-row tiles (4100)."""
    _, (p, s, g) = _fp4_weight(N, K, 700 + N + K)
    x = I.activations("test", 710 + M + K, M, K, "bf16")
    d = dev()
    y = B.fp4_linear(up(x, "bf16"), torch.from_numpy(p).to(d), torch.from_numpy(s).to(d),
                     torch.tensor([g], dtype=torch.float32, device=d))
    _assert_fp4_parity(down(y), x, p, s, g, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K,ng,S", [(300, 1152, None, None), (72, 96, None, None), (1152, 6912, None, None),
                                      (200, 2016, 3, 1), (4100, 1024, 4, 1), (50, 64, 1, 1), (130, 32, 2, 1),
                                      (600, 4640, 2, 3), (64, 20000, 1, None)], ids=str)
def test_fp4_linear_dot_kernel(M, N, K, ng, S, force_plan):
    """The packed-dot kernel for up to four tokens (forced): ragged tail steps
    (96, 32, 4640 = 9 x 512 + 32), K split with the fold, every row-group
    count, K beyond the LDS copy of x (20000: split in at least three)."""
    force_plan("FP4_M4", 2)
    if ng is not None:
        force_plan("FP4_NG", ng)
    if S is not None:
        force_plan("FP4_S", S)
    _, (p, s, g) = _fp4_weight(N, K, 900 + N + K)
    x = I.activations("test", 910 + M + K, M, K, "bf16")
    d = dev()
    y = B.fp4_linear(up(x, "bf16"), torch.from_numpy(p).to(d), torch.from_numpy(s).to(d),
                     torch.tensor([g], dtype=torch.float32, device=d))
    _assert_fp4_parity(down(y), x, p, s, g, f"dot M={M} N={N} K={K} ng={ng} S={S}")


@pytest.mark.parametrize("M", [2, 7])
@pytest.mark.parametrize("ng,S", [(1, 1), (2, 1), (3, 1), (4, 1), (1, 5), (3, 2)])
def test_fp4_linear_tilings(M, ng, S, force_plan):
    """Every compiled row-group count (16 to 64 rows per workgroup) with and
    without a K split, on a ragged N; M = 2 takes the exact per-block kernel
    (up to four tokens), M = 7 the other."""
    force_plan("FP4_NG", ng)
    force_plan("FP4_S", S)
    N, K = 999, 1280
    _, (p, s, g) = _fp4_weight(N, K, 720 + ng)
    x = I.activations("test", 721 + S, M, K, "bf16")
    d = dev()
    y = B.fp4_linear(up(x, "bf16"), torch.from_numpy(p).to(d), torch.from_numpy(s).to(d),
                     torch.tensor([g], dtype=torch.float32, device=d))
    _assert_fp4_parity(down(y), x, p, s, g, f"M={M} NG={ng} S={S}")


@pytest.mark.parametrize("M", [1, 4])
def test_fp4_linear_both_kernels_agree_closely(M, force_plan):
    """Up to four tokens: the exact per-block kernel and the per-weight-rounding
    one against the oracle; the exact one is the closer of the two."""
    N, K = 640, 1152
    _, (p, s, g) = _fp4_weight(N, K, 740 + M)
    x = I.activations("test", 741 + M, M, K, "bf16")
    d = dev()
    args = (torch.from_numpy(p).to(d), torch.from_numpy(s).to(d), torch.tensor([g], dtype=torch.float32, device=d))
    ref = oracle.fp4_linear(x, p, s, g)
    y_exact = down(B.fp4_linear(up(x, "bf16"), *args))
    force_plan("FP4_M4", 0)
    y_round = down(B.fp4_linear(up(x, "bf16"), *args))
    _assert_fp4_parity(y_exact, x, p, s, g, "exact")
    _assert_fp4_parity(y_round, x, p, s, g, "rounded")
    # exact products and fp32 sums: the output rounding and the sums' rounding
    # are all that is left (no 2^-8 per-weight term)
    absref = np.abs(x) @ np.abs(oracle.fp4_unpack(p, s, g)).T
    assert np.all(np.abs(y_exact - ref) <= 2.0 ** -8 * np.abs(ref) * 1.01 + K * 2.0 ** -24 * absref)
    assert rel_err(y_exact, ref) <= rel_err(y_round, ref) + 1e-6


def test_fp4_linear_after_gpu_pack_and_strided_io():
    """Pack on the GPU, then the GEMV with x and y inside wider buffers (ldx > K,
    ldy > N): only the addressed columns of y are written."""
    N, K, M = 640, 1152, 5
    Wb, (p, s, g) = _fp4_weight(N, K, 733)
    d = dev()
    pd, sd, gd = B.quant_fp4_block16(Wb.to(d))
    assert np.array_equal(pd.cpu().numpy(), p) and float(gd.cpu()[0]) == g
    x = I.activations("test", 734, M, K, "bf16")
    xb = torch.zeros((M, K + 64), dtype=torch.bfloat16, device=d)
    xb[:, :K] = up(x, "bf16")
    yb = torch.full((M, N + 24), 3.0, dtype=torch.bfloat16, device=d)
    B.fp4_linear(xb[:, :K], pd, sd, gd, y=yb[:, 8:8 + N])
    got = down(yb)
    assert np.all(got[:, :8] == 3.0) and np.all(got[:, 8 + N:] == 3.0)
    _assert_fp4_parity(got[:, 8:8 + N], x, p, s, g, "strided")


@pytest.mark.parametrize("fam,M", [("gateup", 1), ("gateup", 16), ("down", 4)])
def test_fp4_linear_large_decoder_sampled(fam, M):
    """The large-decoder-shaped weights (stacked gate/up 43008 x 5376; down
    5376 x 21504, K split) on 384 sampled output rows: the GPU pack of the
    whole seeded weight and the GEMV, against the oracle's pack of those rows
    (the weight's largest magnitude is planted in row 0, which every sample
    holds, so the rows' global scale is the whole weight's) and its GEMV."""
    N, K = (43008, 5376) if fam == "gateup" else (5376, 21504)
    rng = np.random.default_rng(4242 + M)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(K ** -0.5)).astype(np.float32)
    W[0, 7] = 1.0                                        # larger than every other |w| (bf16-exact)
    rows = np.concatenate([[0], np.sort(rng.choice(np.arange(1, N), 383, replace=False))])
    d = dev()
    Wb = torch.from_numpy(W).to(torch.bfloat16)        # rounded once, on the host
    del W
    Wr = Wb[torch.from_numpy(rows)].double().numpy()
    Wd = Wb.to(d)
    del Wb
    pd, sd, gd = B.quant_fp4_block16(Wd)
    del Wd
    p, s, g = oracle.fp4_pack(Wr)
    rt = torch.from_numpy(rows).to(d)
    assert float(gd.cpu()[0]) == g
    assert np.array_equal(sd[rt].cpu().numpy(), s) and np.array_equal(pd[rt].cpu().numpy(), p)
    x = I.activations("test", 4300 + M, M, K, "bf16")
    y = down(B.fp4_linear(up(x, "bf16"), pd, sd, gd))
    _assert_fp4_parity(y[:, rows], x, p, s, g, f"{fam} M={M} sampled")


def test_fp4_linear_gemma_stacked_gateup_and_limits():
    """The stacked Gemma-3-1B gate/up weight (13824 x 1152) at M = 16 on
    sampled output columns; M = 0 is a no-op and M = 17 is refused."""
    N, K = 13824, 1152
    Wb, (p, s, g) = _fp4_weight(N, K, 777)
    d = dev()
    pd, sd, gd = torch.from_numpy(p).to(d), torch.from_numpy(s).to(d), torch.tensor([g], dtype=torch.float32, device=d)
    x = I.activations("test", 778, 16, K, "bf16")
    y = down(B.fp4_linear(up(x, "bf16"), pd, sd, gd))
    cols = np.random.default_rng(779).choice(N, 512, replace=False)
    _assert_fp4_parity(y[:, cols], x, p[cols], s[cols], g, "gate/up sampled")
    assert B.fp4_linear(torch.empty((0, K), dtype=torch.bfloat16, device=d), pd, sd, gd).shape == (0, N)
    with pytest.raises(B.AQError):
        B.fp4_linear(up(I.activations("test", 780, 17, K, "bf16"), "bf16"), pd, sd, gd)


# ------------------------------------------------------------- in-graph fold

@pytest.mark.parametrize("M", [16, 300])
def test_fold_path_matches_factored(M):
    """The in-graph fold composed from the library (W_eff materialised into a
    stacked scratch weight, then the GEMM with s = 1 and r = 0) against the
    oracle's factored form: the same y up to the one extra rounding of W_eff."""
    K = 1152
    shapes = [(1024, 64), (256, 64), (256, 64)]
    bds = [I.bundle("test", 9, f, K, n, r, "bf16") for f, (n, r) in zip(("q", "k", "v"), shapes)]
    d = dev()
    weff = torch.cat([B.materialize(bundle_up(b, "bf16")) for b in bds], 0)
    Nt = weff.shape[0]
    ones = torch.ones(Nt, dtype=torch.bfloat16, device=d)
    x = I.activations("test", 990 + M, M, K, "bf16")
    y = B.recon_linear(up(x, "bf16"), (weff, ones, None, None))
    assert_parity(down(y), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16", f"fold M={M}")


# ------------------------------------------------------------- per-element rebuild

def _assert_rebuild_parity(got, x, bds, what):
    """The spec bf16 tolerance against the oracle's factored form, and
    elementwise the bound this arithmetic allows: each rebuilt weight
    s W0 + U Vt formed in fp32 (r + 2 roundings of 2^-24 relative to
    |s W0| + |U| |Vt|) and rounded once to bf16 (2^-8 relative), exact products
    with x, fp32 sums of K terms, one bf16 rounding of y."""
    nb = [bundle_np(b) for b in bds]
    ref = oracle.recon_fused(x, nb)
    assert rel_err(got, ref) <= 1e-2, what
    x64 = np.abs(np.asarray(x, dtype=np.float64))
    A = np.concatenate([np.abs(s)[:, None] * np.abs(W0) + np.abs(U) @ np.abs(Vt) for (W0, s, U, Vt) in nb], 0)
    K = x.shape[1]
    r = max(b[2].shape[1] for b in nb)
    bound = 2.0 ** -8 * np.abs(ref) + (2.0 ** -8 + (r + 2 + K) * 2.0 ** -24) * (x64 @ A.T) * 1.01
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond the derived bound"


@pytest.mark.parametrize("M", [1, 3, 16])
@pytest.mark.parametrize("r", [0, 4, 16, 36, 64])
@pytest.mark.parametrize("variant", ["normal", "s0"])
def test_rebuild_ranks(M, r, variant):
    """Every rank chunk count (r = 0: s W0 only; 4, 16 in one chunk of 32; 36
    and 64 in two, 36 with U rows that are not 16-byte aligned), a ragged N
    (200) and a K that leaves a partial last 32-wide step (1048)."""
    if r == 0 and variant == "s0":
        pytest.skip("s = 0 with r = 0 is the zero map")
    bd, x = _single(M, 1048, 200, r, "bf16", variant=variant, layer=30 + r, tag=3000 + M + r)
    y = B.rebuild_linear(up(x, "bf16"), [bundle_up(bd, "bf16")])
    _assert_rebuild_parity(down(y), x, [bd], f"r={r} M={M} {variant}")


@pytest.mark.parametrize("M", [1, 7, 16])
def test_rebuild_fused_blocks(M):
    """Q/K/V in one dispatch with a rank per block (8, 64, 0): block-diagonal
    U, outputs concatenated along N."""
    K = 264
    shapes = [(200, 8), (40, 64), (24, 0)]
    bds = [I.bundle("test", 31, f, K, n, r, "bf16") for f, (n, r) in zip(("q", "k", "v"), shapes)]
    x = I.activations("test", 3100 + M, M, K, "bf16")
    y = B.rebuild_linear(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    assert y.shape == (M, 264)
    _assert_rebuild_parity(down(y), x, bds, f"qkv M={M}")


@pytest.mark.parametrize("rows,S", [(5, 1), (16, 1), (27, 1), (33, 2), (48, 3), (64, 1), (64, 5), (16, 16)])
def test_rebuild_tilings(rows, S, force_plan):
    """Tiles of any height up to 64 rows (1 to 4 16-row groups, the last tile of
    each block shorter still), with K whole or split over S ranges (fp32
    partials, then the fold), on a ragged gate/up pair."""
    force_plan("REBUILD_ROWS", rows)
    force_plan("REBUILD_S", S)
    K = 1048
    bds = [I.bundle("test", 32, f, K, 333, 16, "bf16") for f in ("gate", "up")]
    x = I.activations("test", 3200 + rows + S, 5, K, "bf16")
    y = B.rebuild_linear(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
    _assert_rebuild_parity(down(y), x, bds, f"rows={rows} S={S}")


@pytest.mark.parametrize("M", [1, 16])
def test_rebuild_gemma_layer_full(M):
    """The Gemma-3-1B-shaped decode layer (rank 16), all four dispatches, every
    output compared."""
    lb = I.layer_bundles("gemma_decode", I.GEMMA_1B, layers=1, r=16, dtype="bf16")[0]
    for name, fams, K, bds in _layer_dispatches(I.GEMMA_1B, lb):
        x = I.activations("gemma_decode", 10 * M + len(name), M, K, "bf16")
        y = B.rebuild_linear(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds])
        _assert_rebuild_parity(down(y), x, bds, f"gemma {name} M={M}")


def test_rebuild_large_decoder_sampled():
    """Large-decoder gate/up and down (rank 32) at M = 4: one output column in
    every 64-column window of every block."""
    lb = I.layer_bundles("large_decoder", I.LARGE_DECODER, layers=1, r=32, dtype="bf16",
                         families=("gate", "up", "down"))[0]
    rng = np.random.default_rng(3300)
    M = 4
    for name, fams in (("gateup", ("gate", "up")), ("down", ("down",))):
        K = I.LARGE_DECODER[fams[0]][0]
        bds = [lb[f] for f in fams]
        x = I.activations("large_decoder", 3300 + len(name), M, K, "bf16")
        y = down(B.rebuild_linear(up(x, "bf16"), [bundle_up(b, "bf16") for b in bds]))
        col0 = 0
        for b in bds:
            n = b["W0"].shape[0]
            cols = _strided_sample(rng, n, 64)
            sb = sub_bundle(b, cols)
            sub = {"W0": sb[0], "s": sb[1], "U": sb[2], "Vt": sb[3]}
            _assert_rebuild_parity(y[:, col0 + cols], x, [sub], f"large {name}")
            col0 += n
        torch.cuda.empty_cache()


def test_rebuild_matches_factored_closely():
    """The rebuild and the factored kernels differ by the one bf16 rounding of
    each rebuilt weight: both within the bound of their own arithmetic, and
    within 2^-7 of max|y| of each other."""
    bd, x = _single(16, 1152, 1024, 16, "bf16", layer=34, tag=3400)
    xd, bdd = up(x, "bf16"), bundle_up(bd, "bf16")
    y_rb = down(B.rebuild_linear(xd, [bdd]))
    y_f = down(B.recon_linear(xd, bdd))
    assert rel_err(y_rb, y_f) <= 2.0 ** -7
