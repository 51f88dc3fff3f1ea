"""Host-side checks of the binding's argument validation and of the load-time
bundle check: every mismatch is reported (all of them, in one exception) before
anything reaches the library.  CPU tensors stand in for device tensors; no
kernel is launched."""

import pytest
import torch

from rank_shared_block_amd import binding as B


def _bundle(N=64, K=128, r=4, dtype=torch.bfloat16):
    return (torch.zeros(N, K, dtype=dtype), torch.ones(N, dtype=dtype),
            torch.zeros(N, r, dtype=dtype), torch.zeros(r, K, dtype=dtype))


def test_recon_reports_every_mismatch_before_the_library():
    W0, s, U, Vt = _bundle()
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError) as e:
        B.recon_linear(x, (W0, s, U, torch.zeros(4, 120, dtype=torch.bfloat16)))
    msg = str(e.value)
    assert "x must be on a GPU" in msg and "Vt must be [4, 128]" in msg
    with pytest.raises(ValueError, match="W0 is \\[64, 128\\] but the input has K = 256"):
        B.recon_linear(torch.zeros(4, 256, dtype=torch.bfloat16), (W0, s, U, Vt))
    with pytest.raises(ValueError, match="s is torch.float32, expected torch.bfloat16"):
        B.recon_linear(x, (W0, s.float(), U, Vt))
    with pytest.raises(ValueError, match="s must be \\[64\\]"):
        B.recon_linear(x, (W0, s[:10], U, Vt))
    with pytest.raises(ValueError, match="U must be \\[64, r\\]"):
        B.recon_linear(x, (W0, s, U[:5], Vt))
    with pytest.raises(ValueError, match="both be given or both be None"):
        B.recon_linear(x, (W0, s, U, None))
    with pytest.raises(ValueError, match="rank 300 exceeds"):
        B.recon_linear(x, (W0, s, torch.zeros(64, 300, dtype=torch.bfloat16),
                           torch.zeros(300, 128, dtype=torch.bfloat16)))
    with pytest.raises(ValueError, match="projection 1: .*W0 is \\[16, 64\\]"):
        B.recon_gateup(x, [(W0, s, U, Vt), _bundle(N=16, K=64)])


def test_other_helpers_validate_their_tensors():
    W0, s, U, Vt = _bundle()
    with pytest.raises(ValueError, match="on a GPU"):
        B.materialize((W0, s, U, Vt))
    with pytest.raises(ValueError, match="on a GPU"):
        B.quant_fp4_block16(W0)
    with pytest.raises(ValueError, match="multiple of 16"):
        B.quant_fp4_block16(torch.zeros(8, 24, dtype=torch.bfloat16))
    x = torch.zeros(2, 128, dtype=torch.bfloat16)
    packed = torch.zeros(32, 64, dtype=torch.uint8)
    scales = torch.zeros(32, 8, dtype=torch.uint8)
    with pytest.raises(ValueError) as e:
        B.fp4_linear(x, packed, scales[:, :4], torch.zeros(2))
    assert "scales must be [32, 8]" in str(e.value) and "one float32 value" in str(e.value)


def _model(L=4, G=2, shapes=(("q", 128, 64), ("down", 256, 32)), r=4):
    shared = {g: {f: torch.zeros(N, K, dtype=torch.bfloat16) for f, K, N in shapes} for g in range(G)}
    layers = {}
    for l in range(L):
        layers[l] = {}
        for f, K, N in shapes:
            _, s, U, Vt = _bundle(N, K, r)
            layers[l][f] = ((l * G) // L, s, U, Vt)
    return shared, layers


def test_check_bundles_accepts_a_consistent_model():
    shared, layers = _model()
    B.check_bundles(shared, layers, require_gpu=False)
    B.check_bundles(shared, layers, quant="nvfp4", require_gpu=False)


def test_check_bundles_lists_every_offending_layer():
    shared, layers = _model(L=6, G=3)
    band, s, U, Vt = layers[1]["q"]
    layers[1]["q"] = (band, s, U, torch.zeros(4, 120, dtype=torch.bfloat16))      # wrong-shaped Vt
    band, s, U, Vt = layers[4]["down"]
    layers[4]["down"] = (band, s, torch.zeros(31, 4, dtype=torch.bfloat16), Vt)   # wrong-shaped U
    layers[5]["q"] = (7,) + layers[5]["q"][1:]                                      # missing band
    _, s, U, Vt = _bundle(64, 128, 300)
    layers[2]["q"] = (1, s, U, Vt)                                                  # r > 256
    with pytest.raises(B.BundleError) as e:
        B.check_bundles(shared, layers, require_gpu=False)
    got = {(l, f) for l, f, _ in e.value.offenders}
    assert got == {(1, "q"), (4, "down"), (5, "q"), (2, "q")}
    msg = str(e.value)
    assert "layer 5 q: band 7 does not exist" in msg
    assert "layer 2 q: rank 300 exceeds" in msg
    assert "layer 1 q: Vt must be [4, 128]" in msg
    assert "layer 4 down: U must be [32, r]" in msg
    assert msg.startswith("4 bundle(s) do not match")


def test_check_bundles_k_divisibility_family_and_device():
    shared, layers = _model(L=2, G=1, shapes=(("o", 100, 48),))
    with pytest.raises(B.BundleError, match="K = 100 must be a multiple of 8"):
        B.check_bundles(shared, layers, require_gpu=False)
    shared, layers = _model(L=2, G=1, shapes=(("o", 136, 48),))
    B.check_bundles(shared, layers, require_gpu=False)
    with pytest.raises(B.BundleError, match="multiple of 16 for the FP4 pack"):
        B.check_bundles(shared, layers, quant="nvfp4", require_gpu=False)
    del shared[0]["o"]
    with pytest.raises(B.BundleError, match="band 0 has no shared block for o"):
        B.check_bundles(shared, layers, require_gpu=False)
    shared, layers = _model(L=2, G=1)
    with pytest.raises(B.BundleError, match="tensors must be on a GPU"):
        B.check_bundles(shared, layers)
    shared[0]["q"] = shared[0]["q"].float()
    with pytest.raises(B.BundleError, match="layer 0 q: W0 is torch.float32, expected torch.bfloat16"):
        B.check_bundles(shared, layers, require_gpu=False)
    with pytest.raises(ValueError, match="unknown quant"):
        B.check_bundles(shared, layers, quant="int4", require_gpu=False)


def test_materialize_model_checks_before_any_launch():
    shared, layers = _model(L=2, G=1)
    layers[1]["q"] = (3,) + layers[1]["q"][1:]
    with pytest.raises(B.BundleError, match="layer 1 q: band 3"):
        B.materialize_model(shared, layers)


def test_debug_plan_knobs():
    assert B.aq_debug_force_plan(len(B.DEBUG_KNOBS), 1) == B.AQ_ERR_INVALID_ARG
    assert "unknown plan knob" in B.last_error()
    B.debug_force_plan("PREFILL_BM", 64)
    B.aq_debug_reset_plan()
    with pytest.raises(ValueError):
        B.debug_force_plan("NO_SUCH_KNOB", 1)


def test_workspace_check_rejects_a_misaligned_workspace():
    # (NULL checks the library's own scratch on the current device: a GPU test)
    assert B.aq_workspace_check(0x10008, None) == B.AQ_ERR_WORKSPACE
    assert "256-byte" in B.last_error()
