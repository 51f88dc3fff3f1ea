"""The allocation-free entry point (aq_recon_linear_noalloc) against the
workspace entry points it stands in for, through the C ABI: the same bits, and
the oracle's result within the bf16 tolerance, on two calls in a row, the second
with a smaller input; decode (streaming kernel, split mode with fp32 partials
in the scratch) and prefill (the rank-r pass handing t over inside one launch,
its counters in the scratch); a call that needs more scratch than the library
holds is refused."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from rank_shared_block_amd import binding as B
from rank_shared_block_amd import inputs as I
from helpers import assert_parity, bundle_np, bundle_up, dev, down, up

pytestmark = pytest.mark.gpu

_FN = {1: "aq_recon_linear", 2: "aq_recon_gateup_fused", 3: "aq_recon_qkv_fused"}


def _both(x, bds, ws):
    """One call of each: (the workspace entry point's y, the no-alloc one's y)."""
    d = dev()
    M, K = x.shape
    projs = [B.make_proj(*b) for b in bds]
    n = len(projs)
    arr = (B.aq_proj * n)(*projs)
    ntot = sum(p.N for p in projs)
    stream = torch.cuda.current_stream().cuda_stream
    y_ws = torch.full((M, ntot), 5.0, dtype=torch.bfloat16, device=d)
    y_na = torch.full((M, ntot), 7.0, dtype=torch.bfloat16, device=d)
    need = B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, M, K, arr, n)
    wsp, wsb = ws.get(need, d)
    B.check(getattr(B.lib(), _FN[n])(B.AQ_BF16, M, K, x.data_ptr(), K, arr, y_ws.data_ptr(), ntot, wsp, wsb, stream))
    B.check(B.aq_recon_linear_noalloc(B.AQ_BF16, M, K, x.data_ptr(), K, list(projs), n, y_na.data_ptr(), ntot, stream))
    torch.cuda.synchronize()
    return y_ws, y_na


@pytest.mark.parametrize("case", ["decode_split", "prefill_handoff", "gemma_layer"])
def test_noalloc_matches_workspace_entry_points(case, force_plan):
    ws = B.Workspace()
    if case == "decode_split":
        # long K: the streaming kernel splits K and keeps fp32 partials in the scratch
        K, shapes, Ms = 6912, [(1152, 16)], (16, 3)
        force_plan("DECODE_SPLIT", 1)
    elif case == "prefill_handoff":
        # 128 x 128 tiles with the rank-r workgroups in the same launch (t and
        # the arrival counters in the scratch)
        K, shapes, Ms = 1048, [(300, 16), (200, 36), (72, 0)], (300, 129)
        for k, v in zip(("BM", "BN", "BK", "NST", "W"), (128, 128, 64, 4, 4)):
            force_plan(f"PREFILL_{k}", v)
    else:
        # the Gemma-3-1B-shaped gate/up dispatch at prefill, default plan
        K, shapes, Ms = 1152, [(6912, 64), (6912, 64)], (2048, 512)
    fams = ("q", "k", "v")[:len(shapes)] if len(shapes) != 2 else ("gate", "up")
    bds = [I.bundle("test", 21, f, K, n, r, "bf16") for f, (n, r) in zip(fams, shapes)]
    dbd = [bundle_up(b, "bf16") for b in bds]
    for i, M in enumerate(Ms):                       # two calls in a row, the second smaller
        x = I.activations("test", 2100 + i, M, K, "bf16")
        y_ws, y_na = _both(up(x, "bf16"), dbd, ws)
        assert torch.equal(y_ws, y_na), f"{case} M={M}: no-alloc and workspace results differ"
        assert_parity(down(y_na), oracle.recon_fused(x, [bundle_np(b) for b in bds]), "bf16", f"{case} M={M}")
    assert B.aq_workspace_check(None, torch.cuda.current_stream().cuda_stream) == B.AQ_OK, B.last_error()
    ws.check()


def test_noalloc_refuses_beyond_its_scratch_and_bad_nproj():
    d = dev()
    # K = 6912 at M = 64 in split mode with 16 splits would need far more than
    # the 16 MiB the library holds: N large, forced split over many K ranges
    K, N, M = 6912, 21504, 64
    W0 = torch.zeros((N, K), dtype=torch.bfloat16, device=d)
    s = torch.ones(N, dtype=torch.bfloat16, device=d)
    x = torch.zeros((M, K), dtype=torch.bfloat16, device=d)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=d)
    p = B.make_proj(W0, s)
    B.debug_force_plan("DECODE_SPLIT", 1)
    B.debug_force_plan("DECODE_S", 16)
    try:
        st = B.aq_recon_linear_noalloc(B.AQ_BF16, M, K, x.data_ptr(), K, [p], 1, y.data_ptr(), N,
                                       torch.cuda.current_stream().cuda_stream)
    finally:
        B.aq_debug_reset_plan()
    assert st == B.AQ_ERR_UNSUPPORTED and "16777216" in B.last_error(), B.last_error()
    assert B.aq_recon_linear_noalloc(B.AQ_BF16, M, K, x.data_ptr(), K, [p], 4, y.data_ptr(), N, None) == \
        B.AQ_ERR_INVALID_ARG
