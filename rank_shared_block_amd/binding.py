"""Thin ctypes binding of ``libaq.so`` (argument marshalling only).

The functions ``aq_*`` mirror the C ABI in ``include/aq.h`` one to one (same
names, same arguments; device pointers and the stream are plain integers).  The
tensor helpers below them only check that the tensors they are given fit
together (device, dtype, shape, layout), turn them into pointers, strides and
the current HIP stream, and raise ``AQError`` for a non-OK status; every step of
the computation runs in the library's HIP kernels.  ``check_bundles`` and
``materialize_model`` are the load-time path: every layer's bundle is checked
against its band's shared block before anything is launched, and one exception
lists every offending layer.  There is no fallback: if the library is missing
or fails to load, every call raises.
"""

import ctypes
import os
import re

import torch   # loaded first: libaq.so then binds to the HIP runtime torch already mapped

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaq.so")

AQ_OK, AQ_ERR_INVALID_ARG, AQ_ERR_SHAPE, AQ_ERR_ALIGNMENT = 0, 1, 2, 3
AQ_ERR_UNSUPPORTED, AQ_ERR_WORKSPACE, AQ_ERR_HIP, AQ_ERR_HANDOFF = 4, 5, 6, 7
AQ_F32, AQ_BF16 = 0, 1
AQ_OP_RECON, AQ_OP_FP4, AQ_OP_FP4_LINEAR, AQ_OP_REBUILD = 0, 1, 2, 3
AQ_MAX_RANK = 256

# Plan overrides (include/aq.h, aq_debug_knob): test-only.
DEBUG_KNOBS = ("DECODE_SPLIT", "DECODE_NG", "DECODE_ROWS", "DECODE_S", "DECODE_WAVES",
               "PREFILL_BM", "PREFILL_BN", "PREFILL_BK", "PREFILL_NST", "PREFILL_W",
               "PREFILL_S", "PREFILL_SELF", "PREFILL_FUSE", "TPASS_S", "TPASS_PARTS",
               "FP4_NG", "FP4_S", "FP4_M4", "HANDOFF_SPIN", "HANDOFF_UNREACHABLE", "REBUILD_NG",
               "REBUILD_ROWS", "REBUILD_S", "MAT_STEPS", "FP4_UNIT", "JACOBI", "JACOBI_WGS")


class aq_proj(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("r", ctypes.c_int64), ("W0", ctypes.c_void_p),
                ("s", ctypes.c_void_p), ("U", ctypes.c_void_p), ("Vt", ctypes.c_void_p)]


class aq_mat_item(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("p", aq_proj), ("w_eff", ctypes.c_void_p), ("ldw", ctypes.c_int64)]


class aq_fp4_item(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("ldw", ctypes.c_int64), ("w", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("global_scale", ctypes.c_void_p)]


class aq_mat_fp4_item(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int64), ("p", aq_proj), ("packed", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p)]


class AQError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        self.detail = detail
        super().__init__(f"{status_string(status)}: {detail}")


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"HIP library not built: {_LIB_PATH} is missing "
                               "(run `python -m rank_shared_block_amd.build`)")
        L = ctypes.CDLL(_LIB_PATH)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        P = ctypes.POINTER(aq_proj)
        for name in ("aq_recon_linear", "aq_recon_qkv_fused", "aq_recon_gateup_fused"):
            f = getattr(L, name)
            f.argtypes = [ctypes.c_int, i64, i64, vp, i64, P, vp, i64, vp, sz, vp]
            f.restype = ctypes.c_int
        L.aq_materialize_weff.argtypes = [ctypes.c_int, i64, P, vp, i64, vp]
        L.aq_materialize_weff.restype = ctypes.c_int
        L.aq_quant_fp4_block16.argtypes = [i64, i64, vp, i64, vp, vp, vp, vp, sz, vp]
        L.aq_quant_fp4_block16.restype = ctypes.c_int
        L.aq_fp4_linear.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, vp, i64, vp, sz, vp]
        L.aq_fp4_linear.restype = ctypes.c_int
        L.aq_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, P, ctypes.c_int]
        L.aq_workspace_bytes.restype = sz
        L.aq_status_string.argtypes = [ctypes.c_int]
        L.aq_status_string.restype = ctypes.c_char_p
        L.aq_last_error.argtypes = []
        L.aq_last_error.restype = ctypes.c_char_p
        L.aq_version.argtypes = []
        L.aq_version.restype = ctypes.c_int
        L.aq_rebuild_linear.argtypes = [ctypes.c_int, i64, i64, vp, i64, P, ctypes.c_int, vp, i64, vp, sz, vp]
        L.aq_rebuild_linear.restype = ctypes.c_int
        L.aq_recon_linear_noalloc.argtypes = [ctypes.c_int, i64, i64, vp, i64, P, ctypes.c_int, vp, i64, vp]
        L.aq_recon_linear_noalloc.restype = ctypes.c_int
        L.aq_band_mean.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(vp), i64, i64, vp, vp]
        L.aq_band_mean.restype = ctypes.c_int
        L.aq_decompose.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.aq_decompose.restype = ctypes.c_int
        L.aq_decompose_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.aq_decompose_workspace_bytes.restype = sz
        L.aq_workspace_check.argtypes = [vp, vp]
        L.aq_workspace_check.restype = ctypes.c_int
        L.aq_debug_force_plan.argtypes = [ctypes.c_int, i64]
        L.aq_debug_force_plan.restype = ctypes.c_int
        L.aq_debug_reset_plan.argtypes = []
        L.aq_debug_reset_plan.restype = None
        L.aq_materialize_batch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(aq_mat_item), vp, vp]
        L.aq_materialize_batch.restype = ctypes.c_int
        L.aq_quant_fp4_batch.argtypes = [ctypes.c_int, ctypes.POINTER(aq_fp4_item), vp, vp, sz, vp]
        L.aq_quant_fp4_batch.restype = ctypes.c_int
        L.aq_quant_fp4_batch_workspace_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.aq_quant_fp4_batch_workspace_bytes.restype = sz
        L.aq_materialize_fp4_batch.argtypes = [ctypes.c_int, ctypes.POINTER(aq_mat_fp4_item), vp, sz, vp]
        L.aq_materialize_fp4_batch.restype = ctypes.c_int
        L.aq_materialize_fp4_batch_workspace_bytes.argtypes = [ctypes.c_int]
        L.aq_materialize_fp4_batch_workspace_bytes.restype = sz
        _lib = L
    return _lib


def library_path():
    return _LIB_PATH


# ----------------------------------------------------------------- raw C ABI

def _projs(p, n):
    if isinstance(p, aq_proj):
        p = [p]
    arr = (aq_proj * n)(*p)
    return arr


def aq_recon_linear(dt, M, K, x, ldx, p, y, ldy, ws, ws_bytes, stream):
    return lib().aq_recon_linear(dt, M, K, x, ldx, _projs(p, 1), y, ldy, ws, ws_bytes, stream)


def aq_recon_qkv_fused(dt, M, K, x, ldx, p, y, ldy, ws, ws_bytes, stream):
    return lib().aq_recon_qkv_fused(dt, M, K, x, ldx, _projs(p, 3), y, ldy, ws, ws_bytes, stream)


def aq_recon_gateup_fused(dt, M, K, x, ldx, p, y, ldy, ws, ws_bytes, stream):
    return lib().aq_recon_gateup_fused(dt, M, K, x, ldx, _projs(p, 2), y, ldy, ws, ws_bytes, stream)


def aq_rebuild_linear(dt, M, K, x, ldx, p, nproj, y, ldy, ws, ws_bytes, stream):
    return lib().aq_rebuild_linear(dt, M, K, x, ldx, _projs(p, nproj), nproj, y, ldy, ws, ws_bytes, stream)


def aq_recon_linear_noalloc(dt, M, K, x, ldx, p, nproj, y, ldy, stream):
    return lib().aq_recon_linear_noalloc(dt, M, K, x, ldx, _projs(p, nproj), nproj, y, ldy, stream)


def aq_materialize_weff(dt, K, p, w_eff, ldw, stream):
    return lib().aq_materialize_weff(dt, K, _projs(p, 1), w_eff, ldw, stream)


def aq_quant_fp4_block16(N, K, w, ldw, packed, scales, global_scale, ws, ws_bytes, stream):
    return lib().aq_quant_fp4_block16(N, K, w, ldw, packed, scales, global_scale, ws, ws_bytes, stream)


def aq_materialize_batch(dt, n, items, amax, stream):
    return lib().aq_materialize_batch(dt, n, items, amax, stream)


def aq_quant_fp4_batch(n, items, amax, ws, ws_bytes, stream):
    return lib().aq_quant_fp4_batch(n, items, amax, ws, ws_bytes, stream)


def aq_quant_fp4_batch_workspace_bytes(n, have_amax):
    return lib().aq_quant_fp4_batch_workspace_bytes(n, have_amax)


def aq_materialize_fp4_batch(n, items, ws, ws_bytes, stream):
    return lib().aq_materialize_fp4_batch(n, items, ws, ws_bytes, stream)


def aq_materialize_fp4_batch_workspace_bytes(n):
    return lib().aq_materialize_fp4_batch_workspace_bytes(n)


def aq_workspace_bytes(op, dt, M, K, p, nproj):
    return lib().aq_workspace_bytes(op, dt, M, K, _projs(p, nproj), nproj)


def aq_band_mean(dt, L, W_ptrs, N, K, W0, stream):
    arr = (ctypes.c_void_p * max(L, 1))(*W_ptrs)
    return lib().aq_band_mean(dt, L, arr, N, K, W0, stream)


def aq_decompose(dt, N, K, r, l, q, W, W0, omega, s, U, Vt, ws, ws_bytes, stream):
    return lib().aq_decompose(dt, N, K, r, l, q, W, W0, omega, s, U, Vt, ws, ws_bytes, stream)


def aq_decompose_workspace_bytes(N, K, r, l):
    return lib().aq_decompose_workspace_bytes(N, K, r, l)


def aq_workspace_check(ws, stream):
    return lib().aq_workspace_check(ws, stream)


def aq_debug_force_plan(knob, value):
    return lib().aq_debug_force_plan(knob, value)


def aq_debug_reset_plan():
    lib().aq_debug_reset_plan()


def debug_force_plan(name, value):
    """Test-only: force one plan knob (a name of DEBUG_KNOBS) on this thread."""
    check(aq_debug_force_plan(DEBUG_KNOBS.index(name), int(value)))


def status_string(s):
    return lib().aq_status_string(s).decode()


def last_error():
    return lib().aq_last_error().decode()


def version():
    return lib().aq_version()


def check(status):
    if status != AQ_OK:
        raise AQError(status, last_error())


# ----------------------------------------------------------- tensor helpers

_DT = {torch.bfloat16: AQ_BF16, torch.float32: AQ_F32}


def _dt(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32") from None


def _ptr(t):
    return t.data_ptr() if (t is not None and t.numel() > 0) else None


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _bundle_problems(W0, s, U, Vt, K=None, dtype=None, device=None):
    """Every way a bundle (W0 [N, K], s [N], U [N, r], Vt [r, K]) fails to fit
    together or to fit (K, dtype, device); an empty list when it fits."""
    bad = []
    if W0 is None or W0.dim() != 2:
        return ["W0 must be a 2-D tensor [N, K]"]
    N, K0 = W0.shape
    if K is not None and K0 != K:
        bad.append(f"W0 is [{N}, {K0}] but the input has K = {K}")
    dtype = W0.dtype if dtype is None else dtype
    device = W0.device if device is None else device
    r = 0 if U is None else (U.shape[1] if U.dim() == 2 else -1)
    if s is None or tuple(s.shape) != (N,):
        bad.append(f"s must be [{N}], got {None if s is None else list(s.shape)}")
    if (U is None) != (Vt is None):
        bad.append("U and Vt must both be given or both be None")
    if U is not None and (U.dim() != 2 or U.shape[0] != N):
        bad.append(f"U must be [{N}, r], got {list(U.shape)}")
    if Vt is not None and U is not None and tuple(Vt.shape) != (max(r, 0), K0):
        bad.append(f"Vt must be [{r}, {K0}] (r from U), got {list(Vt.shape)}")
    if r > AQ_MAX_RANK:
        bad.append(f"rank {r} exceeds the supported maximum {AQ_MAX_RANK}")
    for name, t in (("W0", W0), ("s", s), ("U", U), ("Vt", Vt)):
        if t is None:
            continue
        if t.dtype != dtype:
            bad.append(f"{name} is {t.dtype}, expected {dtype}")
        if t.device != device:
            bad.append(f"{name} is on {t.device}, expected {device}")
        if t.numel() > 0 and not t.is_contiguous():
            bad.append(f"{name} must be contiguous")
    if dtype not in _DT:
        bad.append(f"dtype {dtype} is not bfloat16 or float32")
    elif K0 % (8 if dtype == torch.bfloat16 else 4):
        bad.append(f"K = {K0} must be a multiple of {8 if dtype == torch.bfloat16 else 4} for {dtype}")
    if device.type != "cuda":
        bad.append(f"tensors must be on a GPU, got {device}")
    return bad


def make_proj(W0, s, U=None, Vt=None, K=None, dtype=None, device=None):
    """aq_proj for one bundle of contiguous device tensors (U [N, r], Vt [r, K]);
    raises ValueError listing every mismatch (shapes, dtype, device, layout)."""
    bad = _bundle_problems(W0, s, U, Vt, K, dtype, device)
    if bad:
        raise ValueError("bundle does not fit: " + "; ".join(bad))
    N = W0.shape[0]
    r = 0 if U is None else U.shape[1]
    return aq_proj(N, r, _ptr(W0), _ptr(s), _ptr(U), _ptr(Vt))


class Workspace:
    """A zero-filled device workspace per device, grown on demand.

    The library leaves its counters at zero after every call, so one buffer is
    reused by every call on the stream.  Calls that share it must be ordered on
    one stream.
    """

    def __init__(self):
        self._buf = {}

    def get(self, nbytes, device):
        if nbytes == 0:
            return None, 0
        key = torch.device(device).index
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            size = max(nbytes, 1 << 20)
            buf = torch.zeros(size, dtype=torch.uint8, device=device)
            self._buf[key] = buf
        return buf.data_ptr(), buf.numel()

    def check(self, device=None):
        """aq_workspace_check on this workspace's buffer for `device` (raises
        AQError for a prefill hand-off that gave up, or dirty counters)."""
        key = torch.device(device if device is not None else "cuda").index
        key = torch.cuda.current_device() if key is None else key
        buf = self._buf.get(key)
        if buf is not None:
            check(aq_workspace_check(buf.data_ptr(), _stream()))


_WS = Workspace()


def default_workspace():
    return _WS


def _check_out(y, M, ncols, x, what="y"):
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError(f"{what} must be 2-D with unit column stride")
    if y.shape[0] != M or y.shape[1] < ncols:
        raise ValueError(f"{what} must be [{M}, >= {ncols}], got {list(y.shape)}")
    if y.dtype != x.dtype or y.device != x.device:
        raise ValueError(f"{what} must be {x.dtype} on {x.device}, got {y.dtype} on {y.device}")


def _recon(fn, nproj, x, bundles, y, workspace):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dt = _dt(x)
    M, K = x.shape
    bad = [] if x.device.type == "cuda" else [f"x must be on a GPU, got {x.device}"]
    for i, b in enumerate(bundles):
        for msg in _bundle_problems(*b, K=K, dtype=x.dtype, device=x.device):
            bad.append(f"projection {i}: {msg}")
    if bad:
        raise ValueError("; ".join(bad))
    projs = [make_proj(*b) for b in bundles]
    ntot = sum(p.N for p in projs)
    if y is None:
        y = torch.empty((M, ntot), dtype=x.dtype, device=x.device)
    _check_out(y, M, ntot, x)
    arr = (aq_proj * nproj)(*projs)
    need = lib().aq_workspace_bytes(AQ_OP_RECON, dt, M, K, arr, nproj)
    ws, ws_bytes = (workspace or _WS).get(need, x.device)
    check(fn(dt, M, K, _ptr(x), x.stride(0), arr, _ptr(y), y.stride(0), ws, ws_bytes, _stream()))
    return y


def recon_linear(x, bundle, y=None, workspace=None):
    """y = s * (x W0^T) + (x Vt^T) U^T for bundle = (W0, s, U, Vt)."""
    return _recon(lib().aq_recon_linear, 1, x, [bundle], y, workspace)


def recon_qkv(x, bundles, y=None, workspace=None):
    """[y_q | y_k | y_v] for bundles = (q, k, v), each (W0, s, U, Vt)."""
    if len(bundles) != 3:
        raise ValueError("need three bundles (q, k, v)")
    return _recon(lib().aq_recon_qkv_fused, 3, x, bundles, y, workspace)


def recon_gateup(x, bundles, y=None, workspace=None):
    """[y_gate | y_up] for bundles = (gate, up)."""
    if len(bundles) != 2:
        raise ValueError("need two bundles (gate, up)")
    return _recon(lib().aq_recon_gateup_fused, 2, x, bundles, y, workspace)


def rebuild_linear(x, bundles, y=None, workspace=None):
    """Per-element rebuild: y = x W_eff^T, every weight rebuilt in the kernel;
    bundles = one to three (W0, s, U, Vt) read by the same x, outputs
    concatenated along N (x bf16 [M <= 16, K], r <= 64)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    if not 1 <= len(bundles) <= 3:
        raise ValueError("need one to three bundles")
    M, K = x.shape
    bad = [] if x.device.type == "cuda" else [f"x must be on a GPU, got {x.device}"]
    for i, b in enumerate(bundles):
        for msg in _bundle_problems(*b, K=K, dtype=x.dtype, device=x.device):
            bad.append(f"projection {i}: {msg}")
    if bad:
        raise ValueError("; ".join(bad))
    projs = [make_proj(*b) for b in bundles]
    ntot = sum(p.N for p in projs)
    if y is None:
        y = torch.empty((M, ntot), dtype=x.dtype, device=x.device)
    _check_out(y, M, ntot, x)
    arr = (aq_proj * len(projs))(*projs)
    need = lib().aq_workspace_bytes(AQ_OP_REBUILD, _dt(x), M, K, arr, len(projs))
    ws, ws_bytes = (workspace or _WS).get(need, x.device)
    check(lib().aq_rebuild_linear(_dt(x), M, K, _ptr(x), x.stride(0), arr, len(projs), _ptr(y), y.stride(0),
                                  ws, ws_bytes, _stream()))
    return y


def materialize(bundle, out=None):
    """W_eff = diag(s) W0 + U Vt into `out` (a [N, >=K] view with unit column
    stride; allocated when None)."""
    W0 = bundle[0]
    p = make_proj(*bundle)
    dt = _dt(W0)
    N, K = W0.shape
    if out is None:
        out = torch.empty((N, K), dtype=W0.dtype, device=W0.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != N or out.shape[1] < K:
        raise ValueError(f"out must be [{N}, >= {K}] with unit column stride, got {list(out.shape)}")
    if out.dtype != W0.dtype or out.device != W0.device:
        raise ValueError(f"out must be {W0.dtype} on {W0.device}")
    check(lib().aq_materialize_weff(dt, K, ctypes.byref(p), _ptr(out), out.stride(0), _stream()))
    return out


def quant_fp4_block16(w, workspace=None):
    """Pack a bf16 [N, K] weight; returns (packed uint8 [N, K/2],
    scales uint8 [N, K/16] (E4M3FN bits), global_scale float32 [1])."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D bfloat16 tensor with unit column stride")
    N, K = w.shape
    bad = [] if w.device.type == "cuda" else [f"w must be on a GPU, got {w.device}"]
    if K % 16:
        bad.append(f"K = {K} must be a multiple of 16")
    if bad:
        raise ValueError("; ".join(bad))
    dev = w.device
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty((1,), dtype=torch.float32, device=dev)
    need = lib().aq_workspace_bytes(AQ_OP_FP4, AQ_BF16, 0, K, (aq_proj * 1)(aq_proj(N, 0, None, None, None, None)), 1)
    ws, ws_bytes = (workspace or _WS).get(need, dev)
    check(lib().aq_quant_fp4_block16(N, K, _ptr(w), w.stride(0), _ptr(packed), _ptr(scales),
                                     _ptr(g), ws, ws_bytes, _stream()))
    return packed, scales, g


def materialize_batch(bundles, outs=None, want_amax=False):
    """W_eff for many bundles (W0, s, U, Vt) in a few launches (bf16, r <= 64);
    bundles that name the same W0 tensor next to each other share its reads.
    Returns the list of W_eff (and, with want_amax, the int32 tensor of their
    largest magnitudes as bf16 bits, the input of quant_fp4_batch)."""
    n = len(bundles)
    if n == 0:
        return ([], None) if want_amax else []
    dev = bundles[0][0].device
    outs = list(outs) if outs is not None else [None] * n
    items = (aq_mat_item * n)()
    for i, bd in enumerate(bundles):
        W0 = bd[0]
        N, K = W0.shape
        if outs[i] is None:
            outs[i] = torch.empty((N, K), dtype=W0.dtype, device=W0.device)
        o = outs[i]
        if o.dim() != 2 or o.stride(1) != 1 or o.shape[0] != N or o.shape[1] < K or o.dtype != W0.dtype \
                or o.device != W0.device:
            raise ValueError(f"bundle {i}: out must be {W0.dtype} [{N}, >= {K}] with unit column stride on {W0.device}")
        items[i] = aq_mat_item(K, make_proj(*bd), _ptr(o), o.stride(0))
    amax = torch.empty(n, dtype=torch.int32, device=dev) if want_amax else None
    check(lib().aq_materialize_batch(_dt(bundles[0][0]), n, items, _ptr(amax) if want_amax else None, _stream()))
    return (outs, amax) if want_amax else outs


def quant_fp4_batch(weights, amax=None, workspace=None):
    """FP4 pack of many bf16 [N, K] weights in a few launches; amax (from
    materialize_batch) lets it read each weight once.  Returns a list of
    (packed, scales, global_scale) as quant_fp4_block16."""
    n = len(weights)
    if n == 0:
        return []
    dev = weights[0].device
    items = (aq_fp4_item * n)()
    out = []
    for i, w in enumerate(weights):
        if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1 or w.device != dev:
            raise ValueError(f"weight {i}: must be a 2-D bfloat16 tensor with unit column stride on {dev}")
        N, K = w.shape
        if K % 16:
            raise ValueError(f"weight {i}: K = {K} must be a multiple of 16")
        packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
        g = torch.empty((1,), dtype=torch.float32, device=dev)
        items[i] = aq_fp4_item(N, K, w.stride(0), _ptr(w), _ptr(packed), _ptr(scales), _ptr(g))
        out.append((packed, scales, g))
    if amax is not None and (amax.dtype != torch.int32 or amax.numel() != n or amax.device != dev):
        raise ValueError(f"amax must be an int32 tensor of {n} words on {dev}")
    need = lib().aq_quant_fp4_batch_workspace_bytes(n, 1 if amax is not None else 0)
    ws, ws_bytes = (workspace or _WS).get(need, dev)
    check(lib().aq_quant_fp4_batch(n, items, _ptr(amax) if amax is not None else None, ws, ws_bytes, _stream()))
    return out


def materialize_fp4_batch(bundles, workspace=None):
    """The FP4 weights of many bundles (W0, s, U, Vt; bf16, r <= 64, K % 16
    == 0) without their bf16 W_eff: the bytes of materialize_batch followed by
    quant_fp4_batch.  Returns a list of (packed, scales, global_scale)."""
    n = len(bundles)
    if n == 0:
        return []
    dev = bundles[0][0].device
    items = (aq_mat_fp4_item * n)()
    out = []
    for i, bd in enumerate(bundles):
        N, K = bd[0].shape
        if K % 16:
            raise ValueError(f"bundle {i}: K = {K} must be a multiple of 16")
        packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
        g = torch.empty((1,), dtype=torch.float32, device=dev)
        items[i] = aq_mat_fp4_item(K, make_proj(*bd), _ptr(packed), _ptr(scales), _ptr(g))
        out.append((packed, scales, g))
    need = lib().aq_materialize_fp4_batch_workspace_bytes(n)
    ws, ws_bytes = (workspace or _WS).get(need, dev)
    check(lib().aq_materialize_fp4_batch(n, items, ws, ws_bytes, _stream()))
    return out


def aq_fp4_linear(M, N, K, x, ldx, packed, scales, global_scale, y, ldy, ws, ws_bytes, stream):
    return lib().aq_fp4_linear(M, N, K, x, ldx, packed, scales, global_scale, y, ldy, ws, ws_bytes, stream)


def fp4_linear(x, packed, scales, global_scale, y=None, workspace=None):
    """y = x Wq^T for a packed weight (quant_fp4_block16's outputs), x bf16
    [M <= 16, K]; returns bf16 [M, N]."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 tensor with unit column stride")
    M, K = x.shape
    N = packed.shape[0]
    bad = []
    if packed.dtype != torch.uint8 or scales.dtype != torch.uint8:
        bad.append("packed and scales must be uint8")
    if packed.dim() != 2 or packed.shape[1] * 2 != K:
        bad.append(f"packed must be [N, {K // 2}], got {list(packed.shape)}")
    if tuple(scales.shape) != (N, K // 16):
        bad.append(f"scales must be [{N}, {K // 16}], got {list(scales.shape)}")
    if global_scale.dtype != torch.float32 or global_scale.numel() != 1:
        bad.append("global_scale must be one float32 value")
    if not (packed.is_contiguous() and scales.is_contiguous()):
        bad.append("packed and scales must be contiguous")
    for name, t in (("x", x), ("packed", packed), ("scales", scales), ("global_scale", global_scale)):
        if t.device != x.device or t.device.type != "cuda":
            bad.append(f"{name} must be on the GPU of x, got {t.device}")
    if bad:
        raise ValueError("; ".join(bad))
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _check_out(y, M, N, x)
    need = lib().aq_workspace_bytes(AQ_OP_FP4_LINEAR, AQ_BF16, M, K,
                                    (aq_proj * 1)(aq_proj(N, 0, None, None, None, None)), 1)
    ws, ws_bytes = (workspace or _WS).get(need, x.device)
    check(lib().aq_fp4_linear(M, N, K, _ptr(x), x.stride(0), _ptr(packed), _ptr(scales), _ptr(global_scale),
                              _ptr(y), y.stride(0), ws, ws_bytes, _stream()))
    return y


# ----------------------------------------------------------- decomposition

FULL_SVD_MAX_MIN_DIM = 256      # the pages take a full SVD at or below this min(out, in)


def probe_width(N, K, r, oversample=10):
    """Width l of the randomized SVD's probe for a rank-r truncation of an
    [N, K] residual: r + oversample, or min(N, K) -- the whole matrix, which
    makes the same steps an exact SVD -- where the pages take a full SVD
    (min(N, K) <= 256, or r + oversample >= min(N, K))."""
    m = min(N, K)
    return m if (m <= FULL_SVD_MAX_MIN_DIM or r + oversample >= m) else r + oversample


def band_mean(weights, out=None):
    """W0 = the mean of a band's layer weights (same shape, bf16 or fp32, one
    device), rounded once."""
    W = list(weights)
    if not W:
        raise ValueError("need at least one layer weight")
    w0 = W[0]
    bad = [i for i, w in enumerate(W) if w.shape != w0.shape or w.dtype != w0.dtype or w.device != w0.device
           or w.dim() != 2 or not w.is_contiguous()]
    if bad:
        raise ValueError(f"layer weights {bad} differ from layer 0 in shape, dtype, device or layout")
    if w0.device.type != "cuda":
        raise ValueError(f"weights must be on a GPU, got {w0.device}")
    N, K = w0.shape
    if out is None:
        out = torch.empty_like(w0)
    check(aq_band_mean(_dt(w0), len(W), [w.data_ptr() for w in W], N, K, out.data_ptr(), _stream()))
    return out


def decompose(W, W0, r, omega, q=2, workspace=None):
    """(s, U, Vt) float64 for one weight and its shared block: least-squares
    row scale, then the rank-r truncated SVD of the residual by the randomized
    method with the Gaussian probe `omega` [l, K] (float64, on the GPU) and q
    subspace steps; l = probe_width(...) reproduces the pages' size rule."""
    if W.shape != W0.shape or W.dtype != W0.dtype or W.device != W0.device or W.dim() != 2:
        raise ValueError("W and W0 must be 2-D tensors of one shape, dtype and device")
    if not (W.is_contiguous() and W0.is_contiguous()) or W.device.type != "cuda":
        raise ValueError("W and W0 must be contiguous GPU tensors")
    N, K = W.shape
    dev = W.device
    l = 0 if r == 0 else omega.shape[0]
    if r > 0 and (omega.dtype != torch.float64 or omega.dim() != 2 or omega.shape[1] != K
                  or omega.device != dev or not omega.is_contiguous()):
        raise ValueError(f"omega must be a contiguous float64 [l, {K}] tensor on {dev}")
    s = torch.empty(N, dtype=torch.float64, device=dev)
    U = torch.empty((N, r), dtype=torch.float64, device=dev)
    Vt = torch.empty((r, K), dtype=torch.float64, device=dev)
    need = aq_decompose_workspace_bytes(N, K, r, l) if r > 0 else 0
    ws, ws_bytes = (workspace or _WS).get(need, dev) if need else (None, 0)
    check(aq_decompose(_dt(W), N, K, r, l, q, W.data_ptr(), W0.data_ptr(), _ptr(omega) if r else None,
                       s.data_ptr(), _ptr(U), _ptr(Vt), ws, ws_bytes, _stream()))
    return s, U, Vt


# ----------------------------------------------------------- load-time path

class BundleError(ValueError):
    """A model's bundles do not fit their shared blocks.  ``offenders`` lists
    ``(layer, family, reason)`` for every offending layer."""

    def __init__(self, offenders):
        self.offenders = offenders
        lines = [f"layer {l} {f}: {why}" for l, f, why in offenders]
        super().__init__(f"{len(offenders)} bundle(s) do not match a shape- and band-compatible "
                         "shared block (a band count that differs between decomposition and "
                         "serving is the usual cause):\n  " + "\n  ".join(lines))


def check_bundles(shared, layers, quant=None, require_gpu=True):
    """Validate a whole model before anything is launched.

    ``shared[band][family]`` is the shared block W0 [N, K] of a band;
    ``layers[l][family]`` is ``(band, s, U, Vt)`` (U, Vt None for rank 0).  Each
    layer's bundle must name an existing band whose W0 for that family exists,
    and s [N], U [N, r], Vt [r, K] must fit that W0 (one dtype, one GPU,
    contiguous, r <= 256, K a multiple of 8 for bf16 or 4 for fp32, and of 16
    with ``quant="nvfp4"``).  Raises one BundleError that lists every offending
    layer ("Execution paths", section "Precompute-outside": the precompute
    raises immediately with the offending layers listed).  ``require_gpu=False``
    checks everything but the device type (host-side tests of the check).
    """
    if quant not in (None, "nvfp4"):
        raise ValueError(f"unknown quant {quant!r}")
    bad = []
    dtype = device = None
    for l in sorted(layers):
        for f in sorted(layers[l]):
            entry = layers[l][f]
            if len(entry) != 4:
                bad.append((l, f, "expected (band, s, U, Vt)"))
                continue
            band, s, U, Vt = entry
            if band not in shared:
                bad.append((l, f, f"band {band} does not exist (bands: {sorted(shared)})"))
                continue
            W0 = shared[band].get(f)
            if W0 is None:
                bad.append((l, f, f"band {band} has no shared block for {f}"))
                continue
            dtype = W0.dtype if dtype is None else dtype
            device = W0.device if device is None else device
            for msg in _bundle_problems(W0, s, U, Vt, dtype=dtype, device=device):
                if require_gpu or not msg.startswith("tensors must be on a GPU"):
                    bad.append((l, f, msg))
            if quant == "nvfp4" and W0.dim() == 2 and W0.shape[1] % 16:
                bad.append((l, f, f"K = {W0.shape[1]} must be a multiple of 16 for the FP4 pack"))
    if bad:
        raise BundleError(bad)


def materialize_model(shared, layers, quant=None):
    """The load-time path: ``check_bundles``, then every W_eff, or (with
    ``quant="nvfp4"``) every FP4 weight, without the bf16 W_eff where the
    batched calls take the bundle.  Returns ``{layer: {family: W_eff}}`` or
    ``{layer: {family: (packed, scales, global_scale)}}``."""
    check_bundles(shared, layers, quant)
    # family by family, band by band: the layers of one band sit next to each
    # other, so each of their shared blocks is read once per pair of layers
    order = sorted(((f, layers[l][f][0], l) for l in layers for f in layers[l]), key=lambda k: (k[0], str(k[1]), k[2]))
    batch = [(f, b, l) for f, b, l in order if shared[b][f].dtype == torch.bfloat16
             and (layers[l][f][2] is None or layers[l][f][2].shape[1] <= 64)]
    out = {l: {} for l in layers}
    if batch:
        bundles = [(shared[b][f],) + tuple(layers[l][f][1:]) for f, b, l in batch]
        packs = materialize_fp4_batch(bundles) if quant == "nvfp4" else materialize_batch(bundles)
        for (f, b, l), v in zip(batch, packs):
            out[l][f] = v
    for f, b, l in order:                  # fp32 weights and ranks above 64
        if f not in out[l]:
            band, s, U, Vt = layers[l][f]
            w = materialize((shared[band][f], s, U, Vt))
            out[l][f] = quant_fp4_block16(w) if quant == "nvfp4" else w
    return out


def hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process (expect exactly one)."""
    with open("/proc/self/maps") as f:
        return sorted(set(re.findall(r"\S*libamdhip64\S*", f.read())))
