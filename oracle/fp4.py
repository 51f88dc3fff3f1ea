"""Block-16 FP4 packing of an effective weight, float64 reference.

Test infrastructure only (see the package docstring).

The container comes from "Internals and extension" §Nvfp4Spec: two E2M1 values
per byte, so a logical ``[N, K]`` weight is stored as ``[N, K // 2]`` bytes; every
16 consecutive K-values share one FP8-E4M3 block scale (linear layout
``[N, K // 16]``); one fp32 global scale per tensor.  "Execution paths"
§Precompute-outside says each W_eff is quantised to 4-bit at load.

PARITY UNPINNED BY THE PAGES: the pages give the container, not the recipe.  The
recipe below is this oracle's reading, chosen to be deterministic and exactly
reproducible without a per-element division:

1. ``A = max |W|`` over the whole tensor.  The global scale is the dequantisation
   multiplier ``g = RN_f32(A / (6 * 448))`` (E2M1 max times E4M3 max), or
   ``g = 1`` when ``A == 0``.
2. Per row and per 16-value block, ``a = max |w|`` over the block and the block
   scale is ``sf = E4M3FN(a / (6 g))``: the exact quotient rounded to nearest,
   ties to even, saturating at 448, subnormals kept.
3. The block's step is ``D = RN_f32(g * value(sf))``.  ``D == 0`` gives all-zero
   codes.
4. Each element's magnitude code is the E2M1 grid point nearest to the exact
   quotient ``|w| / D``, ties to the even code, saturating at 6.  The sign bit is
   set only for a negative element with a non-zero magnitude (no negative zero).
5. Nibble order: element ``2i`` goes to the low nibble of byte ``i``, element
   ``2i+1`` to the high nibble.  The scale byte is the E4M3FN bit pattern
   (bias 7, no infinities, 0x7F/0xFF are NaN and never produced).

Exactness of the float64 quotients used below: ``a`` and ``|w|`` are bf16 values
(8 significant bits), ``6 g`` has at most 26 and ``D`` at most 24 significant
bits, and the grids' midpoints have at most 5 (E4M3) or 3 (E2M1) significant
bits.  A quotient that equals a midpoint is representable, so the float64
division returns it exactly; one that does not equal a midpoint differs from it
by a relative amount far above float64's 2**-53, so rounding the quotient to
float64 cannot move it across the midpoint.  The tests check this claim against
exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np

from .rounding import rne_f32, rn_f32_exact

FP4_BLOCK = 16
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def e2m1_decode(code):
    """Value of a 4-bit E2M1 code: 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    code = np.asarray(code, dtype=np.int64)
    sign = np.where(code & 8, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return sign * mag


E2M1_VALUES = e2m1_decode(np.arange(8))          # 0, .5, 1, 1.5, 2, 3, 4, 6


def e4m3fn_decode(bits):
    """Value of an FP8 E4M3FN byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits;
    exponent field 0 is subnormal (m/8 * 2**-6); S.1111.111 is NaN; no infinity."""
    bits = np.asarray(bits, dtype=np.int64)
    sign = np.where(bits & 0x80, -1.0, 1.0)
    e = (bits >> 3) & 0xF
    m = bits & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def _e4m3_grid_round(q):
    """RNE of non-negative float64 values onto the E4M3 grid, saturating at 448."""
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros_like(q)
    nz = q > 0
    _, e = np.frexp(q[nz])                       # q in [2**(e-1), 2**e)
    qexp = np.maximum(e - 4, -9)                 # 3 fraction bits; subnormal step 2**-9
    out[nz] = np.ldexp(np.rint(np.ldexp(q[nz], -qexp)), qexp)
    return np.minimum(out, E4M3_MAX)


def _e4m3_bits_of_value(v):
    """Bit pattern of a non-negative value that lies exactly on the E4M3 grid."""
    v = np.asarray(v, dtype=np.float64)
    bits = np.zeros(v.shape, dtype=np.int64)
    sub = (v > 0) & (v < 2.0 ** -6)
    bits[sub] = np.rint(v[sub] / 2.0 ** -9).astype(np.int64)
    nrm = v >= 2.0 ** -6
    _, e = np.frexp(v[nrm])
    E = e - 1                                    # v in [2**E, 2**(E+1))
    mant = np.rint((v[nrm] / np.exp2(E) - 1.0) * 8).astype(np.int64)
    bits[nrm] = ((E + 7) << 3) | mant
    return bits


def e4m3fn_encode_rne_sat(q):
    """E4M3FN bits of non-negative values: round to nearest, ties to even,
    saturate at 448 (never NaN)."""
    q = np.asarray(q, dtype=np.float64)
    if np.any(q < 0) or not np.all(np.isfinite(q)):
        raise ValueError("block-scale quotients are finite and non-negative")
    return _e4m3_bits_of_value(_e4m3_grid_round(q))


def e2m1_rne_sat(q):
    """Magnitude code (0..7) of the E2M1 grid point nearest to each q >= 0.

    Nearest by absolute distance; on an exact tie the code with an even index
    (an even mantissa bit) wins; anything beyond 6 takes 6.
    """
    q = np.asarray(q, dtype=np.float64)
    dist = np.abs(q[..., None] - E2M1_VALUES)    # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                          # one or two candidates
    codes = np.arange(8)
    even_pick = np.where(cand & (codes % 2 == 0), codes, 99).min(axis=-1)
    any_pick = np.where(cand, codes, 99).min(axis=-1)
    two = cand.sum(axis=-1) > 1
    return np.where(two, even_pick, any_pick).astype(np.int64)


def global_scale(amax):
    """g = RN_f32(A / 2688) from the exact quotient; 1.0 when A == 0."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    return rn_f32_exact(Fraction(amax) / (int(E2M1_MAX) * int(E4M3_MAX)))


def fp4_pack(W):
    """Pack ``W`` ([N, K], bf16 values as float64, K % 16 == 0).

    Returns ``(packed uint8 [N, K//2], scales uint8 [N, K//16], g float)``.
    """
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    if K % FP4_BLOCK:
        raise ValueError("K must be a multiple of 16")
    absW = np.abs(W)
    A = absW.max() if W.size else 0.0
    g = global_scale(A)
    blocks = absW.reshape(N, K // FP4_BLOCK, FP4_BLOCK)
    a = blocks.max(axis=-1)                                  # [N, K/16]
    sf_bits = e4m3fn_encode_rne_sat(a / (6.0 * g))           # 6g exact in fp64
    D = rne_f32(g * e4m3fn_decode(sf_bits))                  # product exact in fp64
    Dfull = np.repeat(D, FP4_BLOCK, axis=1)                  # [N, K]
    safeD = np.where(Dfull > 0, Dfull, 1.0)
    mag = np.where(Dfull > 0, e2m1_rne_sat(absW / safeD), 0)
    code = mag | np.where((W < 0) & (mag != 0), 8, 0)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sf_bits.astype(np.uint8), g


def fp4_unpack(packed, scales, g):
    """Dequantise: value = E2M1(code) * RN_f32(g * E4M3(scale)), float64 [N, K]."""
    packed = np.asarray(packed, dtype=np.int64)
    N, K2 = packed.shape
    codes = np.empty((N, 2 * K2), dtype=np.int64)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    D = rne_f32(float(g) * e4m3fn_decode(np.asarray(scales, dtype=np.int64)))
    return e2m1_decode(codes) * np.repeat(D, FP4_BLOCK, axis=1)


def fp4_linear(x, packed, scales, g):
    """y = x Wq^T, float64 [M, N], with Wq the dequantised block-16 FP4 weight.

    The decode GEMV over a quantised effective weight: "Execution paths"
    §Precompute-outside quantises each W_eff at load and the forward pass then
    uses it in place of the dense weight; the container is "Internals and
    extension" §Nvfp4Spec.  Each weight's value is its E2M1 code's value times
    its block's step ``RN_f32(g * E4M3(scale))`` (``fp4_unpack``); the product with
    ``x`` ([M, K], bf16 values as float64) is exact in float64 up to the
    summation's rounding.  No rounding of the result.
    """
    Wq = fp4_unpack(packed, scales, g)
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != Wq.shape[1]:
        raise ValueError("x must be [M, K] with K = 2 * packed.shape[1]")
    return x @ Wq.T
