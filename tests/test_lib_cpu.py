"""Host-side checks of the C ABI: the library loads, exports every function that
include/aq.h declares, and rejects bad arguments with the documented status
before touching the GPU.  No kernel is launched here."""

import ctypes
import os
import re

import pytest

from rank_shared_block_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aq.h")

FAKE = 0x10000          # a plausible, 256-byte aligned "device pointer" (never dereferenced)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(aq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = _declared()
    assert {"aq_recon_linear", "aq_recon_qkv_fused", "aq_recon_gateup_fused",
            "aq_materialize_weff", "aq_quant_fp4_block16", "aq_fp4_linear", "aq_workspace_bytes",
            "aq_status_string", "aq_last_error", "aq_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_single_hip_runtime_in_process():
    B.lib()
    maps = B.hip_runtimes_mapped()
    assert len(maps) == 1, maps


def test_status_strings_and_version():
    assert B.status_string(B.AQ_ERR_SHAPE) == "AQ_ERR_SHAPE"
    assert B.status_string(99) == "AQ_ERR_UNKNOWN"
    assert B.version() >= 100


def _proj(N=64, r=4, W0=FAKE, s=FAKE, U=FAKE, Vt=FAKE):
    return B.aq_proj(N, r, W0, s, U, Vt)


def _call(**kw):
    a = dict(dt=B.AQ_BF16, M=4, K=128, x=FAKE, ldx=128, p=_proj(), y=FAKE, ldy=64,
             ws=FAKE, ws_bytes=1 << 20, stream=None)
    a.update(kw)
    return B.aq_recon_linear(a["dt"], a["M"], a["K"], a["x"], a["ldx"], a["p"], a["y"],
                             a["ldy"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dt=7), B.AQ_ERR_INVALID_ARG, "dtype"),
    (dict(M=-1), B.AQ_ERR_INVALID_ARG, "negative"),
    (dict(K=0), B.AQ_ERR_SHAPE, "K = 0"),
    (dict(K=100, ldx=100), B.AQ_ERR_ALIGNMENT, "multiple of 8"),
    (dict(ldx=64), B.AQ_ERR_SHAPE, "ldx"),
    (dict(ldx=132), B.AQ_ERR_ALIGNMENT, "ldx"),
    (dict(ldy=63), B.AQ_ERR_SHAPE, "ldy"),
    (dict(p=_proj(N=0)), B.AQ_ERR_SHAPE, "N = 0"),
    (dict(p=_proj(r=-1)), B.AQ_ERR_SHAPE, "negative"),
    (dict(p=_proj(r=257)), B.AQ_ERR_UNSUPPORTED, "rank 257"),
    (dict(p=_proj(U=None)), B.AQ_ERR_INVALID_ARG, "U or Vt"),
    (dict(p=_proj(W0=FAKE + 8)), B.AQ_ERR_ALIGNMENT, "W0"),
    (dict(p=_proj(Vt=FAKE + 2)), B.AQ_ERR_ALIGNMENT, "Vt"),
    (dict(x=FAKE + 4), B.AQ_ERR_ALIGNMENT, "x is not"),
    (dict(x=None), B.AQ_ERR_INVALID_ARG, "x or y"),
    (dict(K=1 << 22, ldx=1 << 22), B.AQ_ERR_UNSUPPORTED, "2^22"),
    # K = 6912 splits K across workgroups, which needs the workspace
    (dict(K=6912, ldx=6912, ws=None), B.AQ_ERR_WORKSPACE, "workspace"),
    (dict(K=6912, ldx=6912, ws_bytes=16), B.AQ_ERR_WORKSPACE, "workspace"),
    (dict(K=6912, ldx=6912, ws=FAKE + 64), B.AQ_ERR_WORKSPACE, "256-byte"),
])
def test_recon_argument_errors(kw, status, needle):
    assert _call(**kw) == status
    assert needle in B.last_error()


def test_rank_zero_allows_null_factors_and_empty_batch_is_noop():
    # M == 0 is a no-op: AQ_OK without touching x, y or the GPU
    assert _call(M=0, x=None, y=None, p=_proj(r=0, U=None, Vt=None)) == B.AQ_OK
    assert _call(M=0, x=None, y=None) == B.AQ_OK


def test_fused_calls_validate_every_block():
    ps = [_proj(N=64), _proj(N=16, r=300), _proj(N=16)]
    st = B.aq_recon_qkv_fused(B.AQ_BF16, 4, 128, FAKE, 128, ps, FAKE, 96, FAKE, 1 << 20, None)
    assert st == B.AQ_ERR_UNSUPPORTED and "projection 1" in B.last_error()
    ps = [_proj(N=64), _proj(N=64)]
    st = B.aq_recon_gateup_fused(B.AQ_BF16, 4, 128, FAKE, 128, ps, FAKE, 127, FAKE, 1 << 20, None)
    assert st == B.AQ_ERR_SHAPE and "ldy" in B.last_error()


def test_workspace_query_is_host_only():
    p1 = [_proj(N=1024, r=16)]
    # a short, wide decode layer needs no workspace; a long-K one splits K and
    # needs the reserved region plus fp32 partials
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 16, 1152, p1, 1) == 0
    ws_dec = B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 16, 6912, [_proj(N=1152, r=16)], 1)
    assert ws_dec % 256 == 0 and ws_dec > 65536
    # prefill: at least a bf16 t buffer of M x (r rounded to 16), except where
    # one round of 64 x 64 or 128 x 128 tiles covers the output (they compute
    # their own t for r <= 64)
    ws_pf = B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 2048, 1152, [_proj(N=6912, r=16)], 1)
    assert ws_pf >= 65536 + 2048 * 16 * 2
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 2048, 1152, [_proj(N=1024, r=72)], 1) >= 65536 + 2048 * 80 * 2
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 512, 1152, p1, 1) == 0
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 2048, 1152, p1, 1) == 0
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_F32, 8, 256, [_proj(N=256)], 1) == 0
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 0, 1152, p1, 1) == 0
    assert B.aq_workspace_bytes(B.AQ_OP_FP4, B.AQ_BF16, 0, 1152, p1, 1) == 65536 + 4096
    assert B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, 4, 100, p1, 1) == 0   # invalid K


def test_materialize_argument_errors():
    def mat(**kw):
        a = dict(dt=B.AQ_BF16, K=128, p=_proj(), w=FAKE, ldw=128)
        a.update(kw)
        return B.aq_materialize_weff(a["dt"], a["K"], a["p"], a["w"], a["ldw"], None)
    assert mat(ldw=120) == B.AQ_ERR_SHAPE
    assert mat(ldw=132) == B.AQ_ERR_ALIGNMENT
    assert mat(K=12, ldw=16) == B.AQ_ERR_ALIGNMENT
    assert mat(p=_proj(r=300)) == B.AQ_ERR_UNSUPPORTED
    assert mat(w=None) == B.AQ_ERR_INVALID_ARG
    assert mat(w=FAKE + 8) == B.AQ_ERR_ALIGNMENT


def test_fp4_argument_errors():
    def q(**kw):
        a = dict(N=32, K=64, w=FAKE, ldw=64, packed=FAKE, scales=FAKE, g=FAKE, ws=FAKE, ws_bytes=65536 + 4096)
        a.update(kw)
        return B.aq_quant_fp4_block16(a["N"], a["K"], a["w"], a["ldw"], a["packed"], a["scales"],
                                      a["g"], a["ws"], a["ws_bytes"], None)
    assert q(K=40, ldw=40) == B.AQ_ERR_ALIGNMENT
    assert q(N=0) == B.AQ_ERR_SHAPE
    assert q(ldw=60) == B.AQ_ERR_SHAPE
    assert q(ws_bytes=100) == B.AQ_ERR_WORKSPACE
    assert q(packed=FAKE + 4) == B.AQ_ERR_ALIGNMENT
    assert q(scales=None) == B.AQ_ERR_INVALID_ARG


def test_batch_argument_errors_name_the_item():
    """The load-time batch calls check every item before any launch and name
    the first offending one."""
    def mat_items(**bad):
        items = (B.aq_mat_item * 3)()
        for i in range(3):
            items[i] = B.aq_mat_item(128, _proj(), FAKE, 128)
        for k, v in bad.items():
            setattr(items[2], k, v)
        return items
    assert B.aq_materialize_batch(B.AQ_BF16, 3, mat_items(ldw=120), None, None) == B.AQ_ERR_SHAPE
    assert B.last_error().startswith("item 2: ")
    assert B.aq_materialize_batch(B.AQ_BF16, 3, mat_items(p=_proj(r=65)), None, None) == B.AQ_ERR_UNSUPPORTED
    assert "item 2" in B.last_error() and "aq_materialize_weff" in B.last_error()
    assert B.aq_materialize_batch(B.AQ_F32, 3, mat_items(), None, None) == B.AQ_ERR_UNSUPPORTED
    assert B.aq_materialize_batch(B.AQ_BF16, -1, mat_items(), None, None) == B.AQ_ERR_INVALID_ARG
    assert B.aq_materialize_batch(B.AQ_BF16, 3, mat_items(), FAKE + 2, None) == B.AQ_ERR_ALIGNMENT
    assert B.aq_materialize_batch(B.AQ_BF16, 0, None, None, None) == B.AQ_OK

    def fp4_items(**bad):
        items = (B.aq_fp4_item * 2)()
        for i in range(2):
            items[i] = B.aq_fp4_item(32, 64, 64, FAKE, FAKE, FAKE, FAKE)
        for k, v in bad.items():
            setattr(items[1], k, v)
        return items
    need = B.aq_quant_fp4_batch_workspace_bytes(2, 0)
    assert need == 65536 + 256 and B.aq_quant_fp4_batch_workspace_bytes(2, 1) == 0
    assert B.aq_quant_fp4_batch(2, fp4_items(K=40, ldw=40), None, FAKE, need, None) == B.AQ_ERR_ALIGNMENT
    assert B.last_error().startswith("item 1: ")
    assert B.aq_quant_fp4_batch(2, fp4_items(), None, FAKE, need - 1, None) == B.AQ_ERR_WORKSPACE
    assert B.aq_quant_fp4_batch(2, fp4_items(), None, None, 0, None) == B.AQ_ERR_WORKSPACE
    assert B.aq_quant_fp4_batch(2, fp4_items(packed=FAKE + 4), FAKE, None, 0, None) == B.AQ_ERR_ALIGNMENT

    def mf_items(**bad):
        items = (B.aq_mat_fp4_item * 3)()
        for i in range(3):
            items[i] = B.aq_mat_fp4_item(128, _proj(), FAKE, FAKE, FAKE)
        for k, v in bad.items():
            setattr(items[2], k, v)
        return items
    need = B.aq_materialize_fp4_batch_workspace_bytes(3)
    assert need == 65536 + 256 and B.aq_materialize_fp4_batch_workspace_bytes(0) == 0
    assert B.aq_materialize_fp4_batch(3, mf_items(K=136), FAKE, need, None) == B.AQ_ERR_ALIGNMENT
    assert B.last_error().startswith("item 2: ") and "multiple of 16" in B.last_error()
    assert B.aq_materialize_fp4_batch(3, mf_items(p=_proj(r=65)), FAKE, need, None) == B.AQ_ERR_UNSUPPORTED
    assert B.last_error().startswith("item 2: ")
    assert B.aq_materialize_fp4_batch(3, mf_items(packed=None), FAKE, need, None) == B.AQ_ERR_INVALID_ARG
    assert B.aq_materialize_fp4_batch(3, mf_items(packed=FAKE + 4), FAKE, need, None) == B.AQ_ERR_ALIGNMENT
    assert B.aq_materialize_fp4_batch(3, mf_items(), FAKE, need - 1, None) == B.AQ_ERR_WORKSPACE
    assert B.aq_materialize_fp4_batch(3, mf_items(), None, 0, None) == B.AQ_ERR_WORKSPACE
    assert B.aq_materialize_fp4_batch(0, None, None, 0, None) == B.AQ_OK


def test_fp4_linear_argument_errors_and_workspace():
    def call(M=1, N=64, K=128, ldx=None, ldy=None, x=FAKE, ptr=FAKE):
        return B.aq_fp4_linear(M, N, K, x, K if ldx is None else ldx, ptr, ptr, ptr, ptr,
                               N if ldy is None else ldy, FAKE, 1 << 20, None)
    assert call(M=17) == B.AQ_ERR_UNSUPPORTED and "16 tokens" in B.last_error()
    assert call(M=-1) == B.AQ_ERR_INVALID_ARG
    assert call(K=48) == B.AQ_ERR_ALIGNMENT
    assert call(K=16) == B.AQ_ERR_SHAPE
    assert call(N=0) == B.AQ_ERR_SHAPE
    assert call(ldx=64) == B.AQ_ERR_SHAPE
    assert call(ldx=132) == B.AQ_ERR_ALIGNMENT
    assert call(ldy=63) == B.AQ_ERR_SHAPE
    assert call(M=0, x=None, ptr=None) == B.AQ_OK                 # no-op, nothing inspected
    assert call(x=None) == B.AQ_ERR_INVALID_ARG
    assert call(x=FAKE + 8) == B.AQ_ERR_ALIGNMENT
    ws = lambda M, N, K: B.aq_workspace_bytes(B.AQ_OP_FP4_LINEAR, B.AQ_BF16, M, K, [_proj(N=N)], 1)
    assert ws(1, 13824, 1152) == 0                                # enough row tiles: no K split
    big = ws(16, 1152, 6912)                                      # few rows, long K: fp32 partials
    assert big > 65536 and (big - 65536) % (16 * 1152 * 4) == 0
    assert ws(17, 64, 128) == 0 and ws(0, 64, 128) == 0


def test_prefill_plans_for_the_gemma_shapes():
    """The planner's choices on the Gemma-3-1B prefill shapes (rank 64), read
    from the workspace each implies: QKV and o tiles compute their own t (no
    workspace); gate/up runs the rank-r pass in its launch with one bf16 t
    [M, 128]; down at M = 512 splits K in three (one t per K range plus fp32
    partials), at M = 2048 keeps K whole with t in two K parts."""
    def ws(M, K, ns):
        arr = (B.aq_proj * len(ns))(*[B.aq_proj(n, r, FAKE, FAKE, FAKE, FAKE) for n, r in ns])
        return B.aq_workspace_bytes(B.AQ_OP_RECON, B.AQ_BF16, M, K, arr, len(ns))
    qkv, o = [(1024, 64), (256, 64), (256, 64)], [(1152, 64)]
    gateup, down = [(6912, 64), (6912, 64)], [(1152, 64)]
    for M in (512, 2048):
        assert ws(M, 1152, qkv) == 0 and ws(M, 1024, o) == 0
        assert ws(M, 1152, gateup) == 65536 + M * 128 * 2
    assert ws(512, 6912, down) == 65536 + 512 * 64 * 2 * 3 + 3 * 512 * 1152 * 4
    assert ws(2048, 6912, down) == 65536 + 2048 * 64 * 2 * 2


def test_rebuild_refusals_before_any_launch():
    def call(dt=B.AQ_BF16, M=4, K=128, ps=None, nproj=1):
        ps = ps or [_proj(N=64, r=16)]
        return B.aq_rebuild_linear(dt, M, K, FAKE, K, ps, nproj, FAKE, 64 * nproj, FAKE, 1 << 20, None)
    assert call(ps=[_proj(r=65)]) == B.AQ_ERR_UNSUPPORTED and "limit 64" in B.last_error()
    assert call(M=17) == B.AQ_ERR_UNSUPPORTED and "16 tokens" in B.last_error()
    assert call(dt=B.AQ_F32) == B.AQ_ERR_UNSUPPORTED and "bf16" in B.last_error()
    assert call(nproj=4, ps=[_proj()] * 4) == B.AQ_ERR_INVALID_ARG
    assert call(K=100) == B.AQ_ERR_ALIGNMENT
    assert call(M=0) == B.AQ_OK
    ws = lambda M, K, N, r: B.aq_workspace_bytes(B.AQ_OP_REBUILD, B.AQ_BF16, M, K, [_proj(N=N, r=r)], 1)
    assert ws(1, 1152, 13824, 16) == 0                       # many rows: whole K per tile
    big = ws(16, 6912, 1152, 16)                             # few rows, long K: fp32 partials
    assert big > 65536 and (big - 65536) % (16 * 1152 * 4) == 0
    assert ws(4, 128, 64, 65) == 0 and ws(17, 128, 64, 4) == 0
