"""Pins for the oracle's block-16 FP4 pack.

The pages fix only the container (two E2M1 codes per byte, an FP8-E4M3 scale per
16 K-values, an fp32 global scale); the quantisation recipe is the oracle's
reading and is pinned here by: the format tables checked against torch's
float8_e4m3fn decoder and conversion, exact rational brute force of every
rounding decision, a hand-worked golden block, round trips and error bounds.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e2m1_table_from_format():
    # 1 sign, 2 exponent bits (bias 1), 1 mantissa bit: the OCP E2M1 value set.
    assert list(oracle.E2M1_VALUES) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(oracle.e2m1_decode(np.arange(8, 16))) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e4m3fn_decode_matches_torch_for_all_256_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    want = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_decode(np.arange(256))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert oracle.e4m3fn_decode(0x7E) == 448.0


def test_e4m3fn_encode_is_inverse_on_grid():
    codes = np.arange(0x7F)                         # every finite non-negative code
    vals = oracle.e4m3fn_decode(codes)
    assert np.array_equal(oracle.e4m3fn_encode_rne_sat(vals), codes)


def test_e4m3fn_encode_matches_torch_rne_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(0, 464, 20000), np.exp2(rng.uniform(-12, 8.8, 20000))])
    v = v[v < 464].astype(np.float32)               # torch does not saturate above 464
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    got = oracle.e4m3fn_encode_rne_sat(v.astype(np.float64))
    assert np.array_equal(got, want)


def test_e4m3fn_saturates_and_ties_to_even():
    assert oracle.e4m3fn_encode_rne_sat(np.array([1e6, 464.0, 500.0])).tolist() == [0x7E] * 3
    # midpoint between 1.0 (0x38) and 1.125 (0x39) goes to the even mantissa 0x38;
    # midpoint between 1.125 and 1.25 (0x3A) goes to 0x3A.
    assert oracle.e4m3fn_encode_rne_sat(np.array([1.0625, 1.1875])).tolist() == [0x38, 0x3A]
    # smallest subnormal 2^-9; half of it ties to zero, three halves ties to 2^-8
    assert oracle.e4m3fn_encode_rne_sat(np.array([2.0 ** -10, 3 * 2.0 ** -10])).tolist() == [0, 2]


# Exact rational brute force of each rounding decision --------------------------

_E4M3_POS = [(c, Fraction(float(oracle.e4m3fn_decode(c)))) for c in range(0x7F)]
_E2M1_POS = [(c, Fraction(float(v))) for c, v in enumerate(oracle.E2M1_VALUES)]


def _nearest_even(q, table):
    """Nearest table entry to the exact rational q; ties -> even code; beyond the
    largest entry -> the largest entry."""
    best = min(abs(q - v) for _, v in table)
    cands = [c for c, v in table if abs(q - v) == best]
    if len(cands) == 2:
        return [c for c in cands if c % 2 == 0][0]
    return cands[0]


def _exact_pack(W):
    N, K = W.shape
    A = max(abs(Fraction(float(w))) for w in W.ravel())
    g = oracle.global_scale(float(A))
    packed = np.zeros((N, K // 2), np.int64)
    scales = np.zeros((N, K // 16), np.int64)
    for n in range(N):
        codes = []
        for b in range(K // 16):
            blk = [Fraction(float(w)) for w in W[n, 16 * b:16 * b + 16]]
            a = max(abs(w) for w in blk)
            sf = _nearest_even(a / (6 * Fraction(g)), _E4M3_POS)
            scales[n, b] = sf
            D = Fraction(oracle.rn_f32_exact(Fraction(g) * Fraction(float(oracle.e4m3fn_decode(sf)))))
            for w in blk:
                if D == 0:
                    codes.append(0)
                    continue
                m = _nearest_even(abs(w) / D, _E2M1_POS)
                codes.append(m | (8 if (w < 0 and m != 0) else 0))
        for i in range(K // 2):
            packed[n, i] = codes[2 * i] | (codes[2 * i + 1] << 4)
    return packed, scales, g


@pytest.mark.parametrize("seed", range(6))
def test_pack_matches_exact_rational_bruteforce(seed):
    rng = np.random.default_rng(seed)
    N, K = 3, 64
    scale = [1e-3, 1.0, 37.0, 2.0 ** -20, 5e3, 0.02][seed]
    W = rng.standard_normal((N, K)) * scale
    W[0, :16] *= 1e-3                               # a block far below the global max
    if seed % 2:
        W[1, 16:32] = 0.0                           # an all-zero block
    W = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    p, s, g = oracle.fp4_pack(W)
    ep, es, eg = _exact_pack(W)
    assert g == eg
    assert np.array_equal(s, es)
    assert np.array_equal(p, ep)


def test_pack_ties_bruteforce():
    """Elements placed exactly on E2M1 midpoints (times D = 1) follow ties-to-even."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    row = [10.5] + [0.0] * 15                       # A = 10.5 -> g = 2^-8 exactly
    row += [6.0] + mids + [-m for m in mids] + [0.0]  # block max 6 -> scale 256, D = 1
    W = np.array([row], dtype=np.float64)
    p, s, g = oracle.fp4_pack(W)
    ep, es, eg = _exact_pack(W)
    assert g == 2.0 ** -8 and s.tolist() == [[0x7E, 0x78]]
    assert np.array_equal(p, ep) and np.array_equal(s, es) and g == eg
    codes = np.empty(32, np.int64)
    codes[0::2] = p[0] & 0xF
    codes[1::2] = p[0] >> 4
    assert codes[17:24].tolist() == [0, 2, 2, 4, 4, 6, 6]        # even-code winners
    assert codes[24:31].tolist() == [0, 10, 10, 12, 12, 14, 14]  # same, negative (no -0)


def test_golden_hand_block():
    with open(os.path.join(GOLDEN, "hand_fp4_block16.json")) as f:
        gd = json.load(f)
    W = np.array(gd["W"], dtype=np.float64)
    p, s, g = oracle.fp4_pack(W)
    assert g == gd["global_scale"]
    assert s.tolist() == gd["scales"]
    assert p.tolist() == gd["packed"]
    codes = np.empty((1, 32), np.int64)
    codes[:, 0::2] = p & 0xF
    codes[:, 1::2] = p >> 4
    assert codes.tolist() == gd["hand_codes"]


def test_round_trip_of_grid_values_is_lossless():
    rng = np.random.default_rng(21)
    N, K = 4, 64
    W = np.zeros((N, K))
    for n in range(N):
        for b in range(K // 16):
            D = 2.0 ** int(rng.integers(-6, 3))          # block step, a power of two
            vals = rng.choice(oracle.E2M1_VALUES, 16) * rng.choice([-1.0, 1.0], 16)
            vals[0] = 6.0                                 # block max = 6 D
            W[n, 16 * b:16 * b + 16] = vals * D
    W[0, :16] = 0.0
    W[0, 0] = 42.0                     # A = 21 * 2: g = 2^-6, so every D above is exact
    p, s, g = oracle.fp4_pack(W)
    assert g == 2.0 ** -6
    back = oracle.fp4_unpack(p, s, g)
    assert np.array_equal(back, W)


def test_dequant_error_bound():
    rng = np.random.default_rng(8)
    W = rng.standard_normal((16, 256)) * np.exp2(rng.uniform(-4, 4, (16, 1)))
    W = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    p, s, g = oracle.fp4_pack(W)
    back = oracle.fp4_unpack(p, s, g)
    D = np.repeat(oracle.rne_f32(g * oracle.e4m3fn_decode(s.astype(np.int64))), 16, axis=1)
    normal = np.repeat(s >= 8, 16, axis=1)                      # block scale not subnormal
    assert normal.mean() > 0.99
    err = np.abs(back - W)
    assert np.all(err[normal] <= D[normal])                     # half the widest gap (2 D)
    small = normal & (np.abs(W) <= 2 * D)
    assert np.all(err[small] <= D[small] / 4)                   # gap 0.5 D below 2 D


def test_all_zero_tensor():
    p, s, g = oracle.fp4_pack(np.zeros((2, 32)))
    assert g == 1.0 and not p.any() and not s.any()


def test_global_scale_exact():
    assert oracle.global_scale(10.5) == 2.0 ** -8
    assert oracle.global_scale(0.0) == 1.0
    # 1/448 is not a binary fraction: compare against exact rational rounding
    g = oracle.global_scale(6.0)
    assert g == oracle.rn_f32_exact(Fraction(6, 2688))
    assert abs(g - 6 / 2688) <= 2.0 ** -24 * (6 / 2688)


# ------------------------------------------------------------------ FP4 GEMV

_E2M1_BY_FORMAT = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}


def _fp4_linear_bruteforce(x, packed, scales, g):
    """Element by element from the container's definition: nibble 2i of byte i
    is the low one; the code value from the E2M1 table; the block step is the
    fp32 product of g and the E4M3 scale (torch's float8_e4m3fn decoder)."""
    N, K2 = packed.shape
    K = 2 * K2
    sv = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    y = np.zeros((x.shape[0], N))
    for n in range(N):
        for k in range(K):
            byte = int(packed[n, k // 2])
            code = (byte >> 4) if k % 2 else (byte & 0xF)
            val = _E2M1_BY_FORMAT[code & 7] * (-1.0 if code & 8 else 1.0)
            step = float(np.float32(g) * np.float32(sv[n, k // 16]))
            for m in range(x.shape[0]):
                y[m, n] += x[m, k] * (val * step)
    return y


@pytest.mark.parametrize("seed", [0, 1])
def test_fp4_linear_matches_bruteforce(seed):
    rng = np.random.default_rng(300 + seed)
    N, K, M = 5, 48, 3
    W = rng.standard_normal((N, K)) * np.exp2(rng.uniform(-3, 3, (N, 1)))
    W = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    p, s, g = oracle.fp4_pack(W)
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    got = oracle.fp4_linear(x, p, s, g)
    want = _fp4_linear_bruteforce(x, p, s, g)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_fp4_linear_one_hot_rows_and_error_bound():
    """A one-hot activation reads one column of the dequantised weight exactly;
    against the unquantised weight the error stays within sum_k |x_k| times the
    elementwise dequantisation bound (the block step D)."""
    rng = np.random.default_rng(44)
    N, K = 24, 128
    W = torch.from_numpy(rng.standard_normal((N, K)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    p, s, g = oracle.fp4_pack(W)
    Wq = oracle.fp4_unpack(p, s, g)
    for k in (0, 17, 127):
        e = np.zeros((1, K))
        e[0, k] = 1.0
        assert np.array_equal(oracle.fp4_linear(e, p, s, g)[0], Wq[:, k])
    x = rng.standard_normal((4, K))
    D = np.repeat(oracle.rne_f32(g * oracle.e4m3fn_decode(s.astype(np.int64))), 16, axis=1)
    err = np.abs(oracle.fp4_linear(x, p, s, g) - x @ W.T)
    assert np.all(err <= np.abs(x) @ D.T)


def test_fp4_linear_zero_codes_give_zero():
    p = np.zeros((3, 16), dtype=np.uint8)
    s = np.full((3, 2), 0x38, dtype=np.uint8)        # scale 1.0
    assert not oracle.fp4_linear(np.ones((2, 32)), p, s, 0.5).any()
    # 0x88: both nibbles are code 8, the negative zero pattern: value 0 too
    assert not oracle.fp4_linear(np.ones((2, 32)), np.full((3, 16), 0x88, dtype=np.uint8), s, 0.5).any()


def _fp4_linear_variants():
    """Plausible mistakes in the FP4 GEMV, each as a whole function: nibble
    order swapped, the sign bit ignored, the block step taken per 32 values,
    the global scale dropped, the weight not transposed (x W instead of x W^T
    on a square case is still wrong)."""
    def unpack_with(packed, scales, g, swap=False, nosign=False, block=16, use_g=True):
        packed = np.asarray(packed, dtype=np.int64)
        N, K2 = packed.shape
        codes = np.empty((N, 2 * K2), dtype=np.int64)
        lo, hi = packed & 0xF, packed >> 4
        codes[:, 0::2], codes[:, 1::2] = (hi, lo) if swap else (lo, hi)
        if nosign:
            codes &= 7
        sv = oracle.e4m3fn_decode(np.asarray(scales, dtype=np.int64))
        D = oracle.rne_f32((float(g) if use_g else 1.0) * sv)
        Dfull = np.repeat(D, 16, axis=1) if block == 16 else np.repeat(D[:, ::2], 32, axis=1)[:, :2 * K2]
        return oracle.e2m1_decode(codes) * Dfull
    return {
        "swapped nibbles": lambda x, p, s, g: x @ unpack_with(p, s, g, swap=True).T,
        "no sign": lambda x, p, s, g: x @ unpack_with(p, s, g, nosign=True).T,
        "32-value blocks": lambda x, p, s, g: x @ unpack_with(p, s, g, block=32).T,
        "no global scale": lambda x, p, s, g: x @ unpack_with(p, s, g, use_g=False).T,
        "not transposed": lambda x, p, s, g: x @ unpack_with(p, s, g),
    }


def _fp4_pins_hold(fn):
    """The GEMV pins above, run against `fn`: brute force, one-hot columns."""
    rng = np.random.default_rng(300)
    N = K = 32
    W = rng.standard_normal((N, K)) * np.exp2(rng.uniform(-3, 3, (N, 1)))
    W = torch.from_numpy(W.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    p, s, g = oracle.fp4_pack(W)
    x = torch.from_numpy(rng.standard_normal((3, K)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    try:
        if not np.allclose(fn(x, p, s, g), _fp4_linear_bruteforce(x, p, s, g), rtol=1e-13, atol=1e-13):
            return False
        Wq = oracle.fp4_unpack(p, s, g)
        e = np.zeros((1, K))
        e[0, 5] = 1.0
        return np.array_equal(fn(e, p, s, g)[0], Wq[:, 5])
    except ValueError:
        return False


def test_fp4_linear_pins_catch_planted_mistakes():
    assert _fp4_pins_hold(oracle.fp4_linear)
    for name, fn in _fp4_linear_variants().items():
        assert not _fp4_pins_hold(fn), f"planted mistake passed the pins: {name}"
