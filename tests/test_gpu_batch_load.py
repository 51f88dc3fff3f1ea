"""GPU parity of the load-time batch calls (aq_materialize_batch,
aq_quant_fp4_batch, aq_materialize_fp4_batch): every W_eff against the oracle's (one rounding; bit-exact
where the rank term is absent), the same bits as the one-projection call, the
largest magnitudes they report, and the FP4 bytes against the oracle's pack.

"Execution paths", section "Precompute-outside" (W_eff rebuilt once at load and
quantised there); "How attnquant works", section "The theta bundle" (the layers
of a band share W0); "Internals and extension", section "Nvfp4Spec" (the
container)."""

import numpy as np
import pytest
import torch

import oracle
from rank_shared_block_amd import binding as B
from rank_shared_block_amd import inputs as I
from helpers import assert_parity, bundle_np, dev, down, up

pytestmark = pytest.mark.gpu


def _band(tag, N, K, ranks, band, variant="normal"):
    """Bundles of len(ranks) layers that share one W0 draw (the same array)."""
    out = []
    for i, r in enumerate(ranks):
        bd = I.bundle("test", 500 + tag * 8 + i, "gate", K, N, r, "bf16", band=900 + band, variant=variant)
        if out:
            bd["W0"] = out[0]["W0"]
        out.append(bd)
    return out


def _upload(bds):
    """Device bundles; the layers of a band get the same W0 tensor."""
    shared, res = {}, []
    for bd in bds:
        k = id(bd["W0"])
        if k not in shared:
            shared[k] = up(bd["W0"], "bf16")
        res.append((shared[k],) + tuple(up(bd[n], "bf16") for n in ("s", "U", "Vt")))
    return res


def _magnitude_max(w):
    """Largest |w| of a bf16 tensor as its bit pattern (bits 0..14)."""
    return int((w.view(torch.int16).to(torch.int32) & 0x7FFF).max())


def _bundles_mixed():
    bds = []
    bds += _band(0, 300, 264, [64, 64], 0)              # a band of two layers, ragged N and K
    bds += _band(1, 130, 1048, [16, 5, 33], 1)          # three layers: a run of two, then one
    bds += _band(2, 77, 64, [0], 2)                     # rank 0
    bds += _band(3, 96, 136, [8, 8], 3, "passthrough")  # s = 1, U = Vt = 0
    bds += _band(4, 1, 8, [40], 4)                      # one row, one 8-wide column block
    for j in range(30):                                 # enough runs and outputs for several launches
        bds += _band(10 + j, 16 + 8 * j, 64 + 16 * (j % 5), [4 * (j % 17), 2 * (j % 9)], 10 + j)
    return bds


def test_materialize_batch_parity_and_same_bits():
    bds = _bundles_mixed()
    dbs = _upload(bds)
    outs, amax = B.materialize_batch(dbs, want_amax=True)
    amax = amax.cpu().numpy()
    assert len(outs) == len(bds) > 48                 # more outputs (and runs) than one launch holds
    for i, (bd, w) in enumerate(zip(bds, outs)):
        ref = oracle.materialize(*bundle_np(bd))
        got = down(w)
        r = bd["U"].shape[1]
        if r == 0 or not np.any(bd["U"]):
            assert np.array_equal(got, oracle.rne_bf16(ref)), f"item {i}: one rounding of s W0"
        else:
            assert_parity(got, ref, "bf16", f"item {i} N={bd['W0'].shape[0]} K={bd['W0'].shape[1]} r={r}")
        assert torch.equal(w, B.materialize(dbs[i])), f"item {i}: not the single call's bits"
        assert amax[i] == _magnitude_max(w), f"item {i}: amax"


@pytest.mark.parametrize("steps", [1, 2, 5])
def test_materialize_batch_unit_lengths(steps, force_plan):
    """Work units of 1, 2 and 5 row steps (the default is 3): the same bits
    (ragged last units included)."""
    bds = _band(70, 700, 200, [24, 64], 70) + _band(71, 129, 72, [7], 71)
    dbs = _upload(bds)
    ref = [B.materialize(d) for d in dbs]
    force_plan("MAT_STEPS", steps)
    outs, amax = B.materialize_batch(dbs, want_amax=True)
    for i, (w, w1) in enumerate(zip(outs, ref)):
        assert torch.equal(w, w1), f"item {i}"
        assert int(amax[i]) == _magnitude_max(w1), f"item {i}: amax"


def test_materialize_batch_strided_outputs_and_empty():
    bds = _band(50, 200, 264, [16, 16], 50)
    dbs = _upload(bds)
    bigs = [torch.full((200 + 6, 264 + 40), -2.0, dtype=torch.bfloat16, device=dev()) for _ in bds]
    B.materialize_batch(dbs, outs=[b[3:203, :] for b in bigs])
    for bd, big in zip(bds, bigs):
        got = down(big)
        assert_parity(got[3:203, :264], oracle.materialize(*bundle_np(bd)), "bf16", "strided")
        assert np.all(got[3:203, 264:] == -2.0) and np.all(got[:3] == -2.0) and np.all(got[203:] == -2.0)
    assert B.materialize_batch([]) == []


def test_materialize_batch_refusals_name_the_item():
    bds = _upload(_band(60, 64, 64, [8, 80], 60))
    with pytest.raises(B.AQError) as e:
        B.materialize_batch(bds)
    assert e.value.status == B.AQ_ERR_UNSUPPORTED and "item 1" in e.value.detail


def _seeded_weights():
    """Pack inputs that do not come from the HIP path: oracle W_eff rounded to
    bf16 (Gemma-shaped k and a few small ones) and a matrix of edge blocks."""
    ws = []
    for j, (N, K, r) in enumerate([(1, 16, 4), (37, 48, 8), (130, 1056, 16), (256, 1152, 64)]):
        bd = I.bundle("test", 700 + j, "k", K, N, r, "bf16")
        ws.append(oracle.rne_bf16(oracle.materialize(*bundle_np(bd))))
    rng = np.random.default_rng(19)
    W = rng.standard_normal((8, 64))
    W[1] = 0.0
    W[2, :16] *= 1e-6
    W[3, 16:32] *= 1e-12
    W[5] = 0.0
    W[5, 0] = 10.5
    W[5, 1:8] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 1.75
    W[0, 0] = 40.0
    ws.append(oracle.rne_bf16(W))
    ws.append(np.zeros((4, 32)))
    for j in range(66):                                 # more weights than one launch holds
        ws.append(oracle.rne_bf16(rng.standard_normal((3 + j, 16 * (1 + j % 4))) * (0.5 + j)))
    return ws


@pytest.mark.parametrize("with_amax,bpt", [(False, None), (True, None), (True, 1), (False, 4), (True, 8)])
def test_quant_fp4_batch_bit_exact(with_amax, bpt, force_plan):
    if bpt is not None:
        force_plan("FP4_UNIT", bpt)
    wn = _seeded_weights()
    wd = [up(w, "bf16") for w in wn]
    amax = None
    if with_amax:            # the inputs' largest magnitudes, written out from their bits
        bits = [int((np.abs(w).astype(np.float32).view(np.uint32) >> 16).max()) for w in wn]
        amax = torch.tensor(bits, dtype=torch.int32, device=dev())
    packs = B.quant_fp4_batch(wd, amax)
    for i, (w, (p, s, g)) in enumerate(zip(wn, packs)):
        ep, es, eg = oracle.fp4_pack(w)
        assert float(g.cpu()[0]) == eg, f"weight {i}: global scale"
        assert np.array_equal(s.cpu().numpy(), es), f"weight {i}: scales"
        assert np.array_equal(p.cpu().numpy(), ep), f"weight {i}: codes"


def test_load_time_chain_gemma_band():
    """Two layers of one band, the seven Gemma-3-1B-shaped families at rank 64:
    the batched materialisation (W0 read once per band) and the pack that takes
    its maxima give the bits of the one-call path, and W_eff is within the
    tolerance of the oracle's."""
    layer_np = I.layer_bundles("materialize_fp4", I.GEMMA_1B, layers=2, r=64, dtype="bf16", num_bands=1)
    bds = [layer_np[l][f] for f in I.FAMILIES for l in (0, 1)]
    dbs = _upload(bds)
    outs, amax = B.materialize_batch(dbs, want_amax=True)
    packs = B.quant_fp4_batch(outs, amax)
    for i, (db, w, (p, s, g)) in enumerate(zip(dbs, outs, packs)):
        w1 = B.materialize(db)
        assert torch.equal(w, w1), f"item {i}: W_eff bits"
        p1, s1, g1 = B.quant_fp4_block16(w1)
        assert torch.equal(p, p1) and torch.equal(s, s1) and torch.equal(g, g1), f"item {i}: pack bytes"
    for i in (0, 9, 13):                       # q of layer 0, gate and down of layer 1, against the oracle
        assert_parity(down(outs[i]), oracle.materialize(*bundle_np(bds[i])), "bf16", f"item {i}")
    for i, ((p, s, g), (p1, s1, g1)) in enumerate(zip(B.materialize_fp4_batch(dbs), packs)):
        assert torch.equal(p, p1) and torch.equal(s, s1) and torch.equal(g, g1), f"item {i}: FP4 without W_eff"


def test_materialize_fp4_batch_same_bytes():
    """aq_materialize_fp4_batch (W_eff formed twice, never stored): the same
    codes, scales and global scales as the batched materialisation followed by
    the batched pack with its maxima, on bundles with K % 16 == 0 -- runs of
    two layers on one W0, ragged N, rank 0, a passthrough bundle, a one-row
    weight, more items than one launch holds."""
    bds = []
    bds += _band(80, 300, 272, [64, 64], 80)
    bds += _band(81, 130, 1056, [16, 5, 33], 81)
    bds += _band(82, 77, 64, [0], 82)
    bds += _band(83, 96, 144, [8, 8], 83, "passthrough")
    bds += _band(84, 1, 16, [40], 84)
    for j in range(28):
        bds += _band(90 + j, 16 + 8 * j, 64 + 16 * (j % 5), [4 * (j % 17), 2 * (j % 9)], 90 + j)
    dbs = _upload(bds)
    assert len(dbs) > 48
    outs, amax = B.materialize_batch(dbs, want_amax=True)
    ref = B.quant_fp4_batch(outs, amax)
    got = B.materialize_fp4_batch(dbs)
    for i, ((p, sc, g), (p1, s1, g1)) in enumerate(zip(got, ref)):
        assert torch.equal(g, g1), f"item {i}: global scale"
        assert torch.equal(sc, s1), f"item {i}: scales"
        assert torch.equal(p, p1), f"item {i}: codes"
    # and the oracle's pack of the oracle's W_eff where W_eff is exact (rank 0
    # and passthrough: one rounding of s W0)
    for i in (5, 6, 7):
        bd = bds[i]
        if bd["U"].shape[1] == 0 or not np.any(bd["U"]):
            ep, es, eg = oracle.fp4_pack(oracle.rne_bf16(oracle.materialize(*bundle_np(bd))))
            p, sc, g = got[i]
            assert float(g.cpu()[0]) == eg and np.array_equal(sc.cpu().numpy(), es) and \
                np.array_equal(p.cpu().numpy(), ep), f"item {i}: oracle"


def test_materialize_model_uses_the_batch_and_falls_back():
    """materialize_model over bands, with one family at a rank above the batch
    limit (the one-projection kernels take it): the result of every layer is
    the one-call path's, packed or not."""
    shapes = {"q": (256, 192), "o": (192, 256)}
    L, G = 4, 2
    bands = [(l * G) // L for l in range(L)]
    rng_r = {"q": 16, "o": 96}
    layer_np = {l: {f: I.bundle("test", 40 + l, f, shapes[f][0], shapes[f][1], rng_r[f], "bf16", band=200 + bands[l])
                    for f in shapes} for l in range(L)}
    shared = {b: {f: up(layer_np[bands.index(b)][f]["W0"], "bf16") for f in shapes} for b in set(bands)}
    layers = {l: {f: (bands[l],) + tuple(up(layer_np[l][f][k], "bf16") for k in ("s", "U", "Vt")) for f in shapes}
              for l in range(L)}
    plain = B.materialize_model(shared, layers)
    packed = B.materialize_model(shared, layers, quant="nvfp4")
    for l in range(L):
        for f in shapes:
            w1 = B.materialize((shared[bands[l]][f],) + layers[l][f][1:])
            assert torch.equal(plain[l][f], w1), f"layer {l} {f}"
            for a, b in zip(packed[l][f], B.quant_fp4_block16(w1)):
                assert torch.equal(a, b), f"layer {l} {f} pack"
