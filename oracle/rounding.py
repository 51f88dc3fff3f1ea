"""Single round-to-nearest-even of float64 values onto narrower binary grids.

Test infrastructure only (see the package docstring).

Written from the formats' definitions (IEEE-754 binary32; bfloat16 = binary32's
exponent range with 8 significant bits).  A finite value x = m * 2**e with
0.5 <= |m| < 1 lies in a binade whose spacing is 2**(e - p) for a format with p
significant bits, floored at the subnormal spacing.  Scaling by a power of two is
exact in float64 and ``np.rint`` rounds half to even, so one call gives one
correctly rounded result.  Overflow is not handled (the workloads stay far inside
the range); the functions raise if a result would overflow.
"""

from fractions import Fraction

import numpy as np

_BF16_P, _BF16_MIN_Q = 8, -133      # 8 significant bits; subnormal spacing 2^-133
_F32_P, _F32_MIN_Q = 24, -149       # 24 significant bits; subnormal spacing 2^-149
_BF16_MAX = float(np.float32(3.3895313892515355e38))
_F32_MAX = float(np.finfo(np.float32).max)


def _rne_grid(x, p, min_q, vmax):
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input")
    _, e = np.frexp(x[nz])
    q = np.maximum(e - p, min_q)
    out[nz] = np.ldexp(np.rint(np.ldexp(x[nz], -q)), q)
    if np.any(np.abs(out) > vmax):
        raise OverflowError("value rounds outside the format's finite range")
    return out


def rne_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even); float64 out."""
    return _rne_grid(x, _BF16_P, _BF16_MIN_Q, _BF16_MAX)


def rne_f32(x):
    """Round float64 values to the nearest binary32 (ties to even); float64 out."""
    return _rne_grid(x, _F32_P, _F32_MIN_Q, _F32_MAX)


def rn_f32_exact(q: Fraction) -> float:
    """Round an exact rational to the nearest binary32 value (ties to even).

    Integer arithmetic only, so there is no intermediate rounding at all.  Used
    where the definition is 'the exact quotient, rounded once to fp32'.
    """
    q = Fraction(q)
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    # e such that 2**(e-1) <= a < 2**e
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** (e - 1) > a:
        e -= 1
    while Fraction(2) ** e <= a:
        e += 1
    qexp = max(e - _F32_P, _F32_MIN_Q)
    scaled = a / (Fraction(2) ** qexp)          # exact
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = fl * (Fraction(2) ** qexp)
    if val > _F32_MAX:
        raise OverflowError("value rounds outside the binary32 range")
    return sign * float(val)
