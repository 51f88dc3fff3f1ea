"""Thin ctypes binding of ``libaq.so`` (argument marshalling only).

The functions ``aq_*`` mirror the C ABI in ``include/aq.h`` one to one (same
names, same arguments; device pointers and the stream are plain integers).  The
tensor helpers below them only turn torch tensors into pointers, strides and the
current HIP stream and raise ``AQError`` for a non-OK status; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or fails to load, every call raises.
"""

import ctypes
import os
import re

import torch   # loaded first: libaq.so then binds to the HIP runtime torch already mapped

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libaq.so")

AQ_OK, AQ_ERR_INVALID_ARG, AQ_ERR_SHAPE, AQ_ERR_ALIGNMENT = 0, 1, 2, 3
AQ_ERR_UNSUPPORTED, AQ_ERR_WORKSPACE, AQ_ERR_HIP = 4, 5, 6
AQ_F32, AQ_BF16 = 0, 1
AQ_OP_RECON, AQ_OP_FP4, AQ_OP_FP4_LINEAR = 0, 1, 2
AQ_MAX_RANK = 256


class aq_proj(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("r", ctypes.c_int64), ("W0", ctypes.c_void_p),
                ("s", ctypes.c_void_p), ("U", ctypes.c_void_p), ("Vt", ctypes.c_void_p)]


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


def aq_materialize_weff(dt, K, p, w_eff, ldw, stream):
    return lib().aq_materialize_weff(dt, K, _projs(p, 1), w_eff, ldw, stream)


def aq_quant_fp4_block16(N, K, w, ldw, packed, scales, global_scale, ws, ws_bytes, stream):
    return lib().aq_quant_fp4_block16(N, K, w, ldw, packed, scales, global_scale, ws, ws_bytes, stream)


def aq_workspace_bytes(op, dt, M, K, p, nproj):
    return lib().aq_workspace_bytes(op, dt, M, K, _projs(p, nproj), nproj)


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


def make_proj(W0, s, U=None, Vt=None):
    """aq_proj for one bundle of contiguous device tensors (U [N, r], Vt [r, K])."""
    N = W0.shape[0]
    r = 0 if U is None else U.shape[1]
    for name, t in (("W0", W0), ("s", s), ("U", U), ("Vt", Vt)):
        if t is not None and t.numel() > 0 and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
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


_WS = Workspace()


def default_workspace():
    return _WS


def _recon(fn, nproj, x, bundles, y, workspace):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dt = _dt(x)
    projs = [make_proj(*b) for b in bundles]
    M, K = x.shape
    ntot = sum(p.N for p in projs)
    if y is None:
        y = torch.empty((M, ntot), dtype=x.dtype, device=x.device)
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be 2-D with unit column stride")
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


def materialize(bundle, out=None):
    """W_eff = diag(s) W0 + U Vt into `out` (a [N, >=K] view with unit column
    stride; allocated when None)."""
    W0 = bundle[0]
    dt = _dt(W0)
    N, K = W0.shape
    if out is None:
        out = torch.empty((N, K), dtype=W0.dtype, device=W0.device)
    if out.dim() != 2 or out.stride(1) != 1 or out.shape[0] != N:
        raise ValueError("out must be [N, >=K] with unit column stride")
    p = make_proj(*bundle)
    check(lib().aq_materialize_weff(dt, K, ctypes.byref(p), _ptr(out), out.stride(0), _stream()))
    return out


def quant_fp4_block16(w, workspace=None):
    """Pack a bf16 [N, K] weight; returns (packed uint8 [N, K/2],
    scales uint8 [N, K/16] (E4M3FN bits), global_scale float32 [1])."""
    if w.dtype != torch.bfloat16 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be a 2-D bfloat16 tensor with unit column stride")
    N, K = w.shape
    dev = w.device
    packed = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
    g = torch.empty((1,), dtype=torch.float32, device=dev)
    need = lib().aq_workspace_bytes(AQ_OP_FP4, AQ_BF16, 0, K, (aq_proj * 1)(aq_proj(N, 0, None, None, None, None)), 1)
    ws, ws_bytes = (workspace or _WS).get(need, dev)
    check(lib().aq_quant_fp4_block16(N, K, _ptr(w), w.stride(0), _ptr(packed), _ptr(scales),
                                     _ptr(g), ws, ws_bytes, _stream()))
    return packed, scales, g


def aq_fp4_linear(M, N, K, x, ldx, packed, scales, global_scale, y, ldy, ws, ws_bytes, stream):
    return lib().aq_fp4_linear(M, N, K, x, ldx, packed, scales, global_scale, y, ldy, ws, ws_bytes, stream)


def fp4_linear(x, packed, scales, global_scale, y=None, workspace=None):
    """y = x Wq^T for a packed weight (quant_fp4_block16's outputs), x bf16
    [M <= 16, K]; returns bf16 [M, N]."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bfloat16 tensor with unit column stride")
    M, K = x.shape
    N = packed.shape[0]
    if packed.shape[1] * 2 != K or scales.shape != (N, K // 16):
        raise ValueError("packed must be [N, K/2] and scales [N, K/16]")
    if not (packed.is_contiguous() and scales.is_contiguous()):
        raise ValueError("packed and scales must be contiguous")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if y.dim() != 2 or y.stride(1) != 1:
        raise ValueError("y must be 2-D with unit column stride")
    need = lib().aq_workspace_bytes(AQ_OP_FP4_LINEAR, AQ_BF16, M, K,
                                    (aq_proj * 1)(aq_proj(N, 0, None, None, None, None)), 1)
    ws, ws_bytes = (workspace or _WS).get(need, x.device)
    check(lib().aq_fp4_linear(M, N, K, _ptr(x), x.stride(0), _ptr(packed), _ptr(scales), _ptr(global_scale),
                              _ptr(y), y.stride(0), ws, ws_bytes, _stream()))
    return y


def hip_runtimes_mapped():
    """Paths of every libamdhip64 mapped into this process (expect exactly one)."""
    with open("/proc/self/maps") as f:
        return sorted(set(re.findall(r"\S*libamdhip64\S*", f.read())))
