"""Pins for the oracle's rounding helpers against library conversions."""

from fractions import Fraction

import numpy as np
import torch

import oracle


def test_rne_bf16_matches_torch_on_f32_inputs():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000) * np.exp2(rng.uniform(-30, 30, 100000)),
                        np.float32(rng.standard_normal(1000)) * np.float32(2.0 ** -128)])
    v32 = v.astype(np.float32)
    want = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.rne_bf16(v32.astype(np.float64)), want)


def test_rne_f32_matches_numpy_cast():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(200000) * np.exp2(rng.uniform(-140, 100, 200000))
    assert np.array_equal(oracle.rne_f32(v), v.astype(np.float32).astype(np.float64))


def test_rn_f32_exact_matches_numpy_on_doubles():
    rng = np.random.default_rng(2)
    for v in rng.standard_normal(2000) * np.exp2(rng.uniform(-60, 60, 2000)):
        assert oracle.rn_f32_exact(Fraction(float(v))) == float(np.float32(v))
    # exact ties: 1 + 2^-24 is halfway between 1 and 1 + 2^-23 -> even (1.0)
    assert oracle.rn_f32_exact(Fraction(1) + Fraction(1, 2 ** 24)) == 1.0
    assert oracle.rn_f32_exact(Fraction(1) + Fraction(3, 2 ** 24)) == 1.0 + 2.0 ** -22
