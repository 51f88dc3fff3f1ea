"""The seeded input generator: deterministic, exact in its dtype, right shapes
and distributions.  It holds no arithmetic of the method."""

import numpy as np
import torch

from rank_shared_block_amd import inputs


def test_deterministic_and_distinct():
    a = inputs.bundle("test", 0, "q", 64, 32, 4, "bf16")
    b = inputs.bundle("test", 0, "q", 64, 32, 4, "bf16")
    c = inputs.bundle("test", 1, "q", 64, 32, 4, "bf16")
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["U"], c["U"])
    assert a["W0"].shape == (32, 64) and a["s"].shape == (32,)
    assert a["U"].shape == (32, 4) and a["Vt"].shape == (4, 64)


def test_bf16_values_are_exact_and_rounded_to_nearest():
    a = inputs.bundle("test", 0, "gate", 128, 256, 8, "bf16")
    for v in a.values():
        assert not np.any(v.view(np.uint32) & 0xFFFF)
    raw = np.random.default_rng(5).standard_normal(10000).astype(np.float32)
    want = torch.from_numpy(raw).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(inputs.round_to_bf16(raw), want)


def test_distributions():
    K, N = 1152, 1024
    b = inputs.bundle("test", 3, "q", K, N, 16, "f32")
    assert abs(b["W0"].std() * np.sqrt(K) - 1) < 0.02
    assert 0.9 <= b["s"].min() and b["s"].max() <= 1.1
    assert abs(b["U"].std() / 0.02 - 1) < 0.05 and abs(b["Vt"].std() / 0.02 - 1) < 0.05
    x = inputs.activations("test", 0, 64, K, "f32")
    assert abs(x.std() - 1) < 0.02


def test_variants_and_bands():
    p = inputs.bundle("test", 0, "o", 64, 32, 4, "f32", variant="passthrough")
    assert np.all(p["s"] == 1) and not p["U"].any() and not p["Vt"].any()
    r0 = inputs.bundle("test", 0, "o", 64, 32, 4, "f32", variant="r0")
    assert r0["U"].shape == (32, 0) and r0["Vt"].shape == (0, 64)
    s0 = inputs.bundle("test", 0, "o", 64, 32, 4, "f32", variant="s0")
    assert not s0["s"].any()
    lb = inputs.layer_bundles("test", {"q": (64, 32), "o": (32, 64)}, layers=4, r=2,
                              dtype="bf16", num_bands=2, families=("q", "o"))
    assert lb[0]["q"]["W0"] is lb[1]["q"]["W0"]
    assert not np.array_equal(lb[1]["q"]["W0"], lb[2]["q"]["W0"])
    assert not np.array_equal(lb[0]["q"]["U"], lb[1]["q"]["U"])


def test_decomposition_inputs_are_seeded_and_banded():
    from rank_shared_block_amd import inputs as I
    a = I.trained_weight("decompose", 0, "q", 256, 96, "bf16", band=0)
    b = I.trained_weight("decompose", 0, "q", 256, 96, "bf16", band=0)
    c = I.trained_weight("decompose", 1, "q", 256, 96, "bf16", band=0)
    assert a.shape == (96, 256) and np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(a, I.round_to_bf16(a))
    # layers of one band share the W0 draw: strongly correlated rows
    cor = np.corrcoef(a.ravel(), c.ravel())[0, 1]
    assert cor > 0.8
    om = I.gaussian_probe("decompose", 3, 12, 256)
    assert om.shape == (12, 256) and om.dtype == np.float64
    assert np.array_equal(om, I.gaussian_probe("decompose", 3, 12, 256))
