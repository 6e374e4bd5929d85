"""Pins of the oracle's number formats against first principles and library casts."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats
from tests.exact import rn_fp16, rn_e4m3_sat


def test_fp16_cast_is_rne_with_subnormals(rng):
    # random fp32 values over the whole fp16 range incl. subnormals, plus exact ties
    x = np.concatenate([
        (rng.standard_normal(4000) * 10.0 ** rng.integers(-8, 4, 4000)).astype(np.float32),
        # ties: midpoints between consecutive fp16 values are exact in fp32
        ((np.arange(1, 2000, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -24)),
        ((np.arange(1024, 2048, dtype=np.float32) + np.float32(0.5)) * np.float32(2.0 ** -10)),
    ])
    got = formats.to_fp16(x).astype(np.float64)
    for xi, gi in zip(x, got):
        assert Fraction(gi) == rn_fp16(Fraction(float(xi))), xi


def test_e4m3_decode_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.e4m3_decode(codes)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_e4m3_encode_matches_torch_in_range(rng):
    x = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 2, 20000),
        np.linspace(-2 ** -6, 2 ** -6, 4001),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.e4m3_encode_rne_sat(x)
    # torch encodes -0 for tiny negatives; the layer's rule maps them to +0
    ref = np.where(ref == 0x80, 0, ref)
    assert np.array_equal(got, ref)


def test_e4m3_encode_against_exact_rounding(rng):
    x = np.concatenate([rng.uniform(0, 500, 3000), rng.uniform(0, 0.05, 3000),
                        # exact midpoints between neighbouring codes
                        (formats.e4m3_decode(np.arange(0, 0x7E)) + formats.e4m3_decode(np.arange(1, 0x7F))) / 2])
    x = x.astype(np.float32)
    got = formats.e4m3_decode(formats.e4m3_encode_rne_sat(x))
    for xi, gi in zip(x, got):
        assert Fraction(gi) == rn_e4m3_sat(Fraction(float(xi)))


def test_e4m3_saturates():
    x = np.array([448.0, 449.0, 464.0, 465.0, 1e6, -1e6], np.float32)
    assert list(formats.e4m3_encode_rne_sat(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e2m1_table():
    vals = formats.e2m1_decode(np.arange(16))
    assert list(vals) == [0, 0.5, 1, 1.5, 2, 3, 4, 6, 0, -0.5, -1, -1.5, -2, -3, -4, -6]


@pytest.mark.parametrize("t,expect", [
    (0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0),
    (0.2499, 0.0), (0.2501, 0.5), (0.7499, 0.5), (2.51, 3.0), (4.99, 4.0), (5.01, 6.0), (100.0, 6.0),
    (-0.25, 0.0), (-0.75, -1.0), (-5.0, -4.0), (-7.0, -6.0),
])
def test_e2m1_ties_and_saturation(t, expect):
    assert formats.e2m1_decode(formats.e2m1_encode(np.array([t])))[0] == expect


def test_e2m1_minus_zero_is_plus_zero():
    assert formats.e2m1_encode(np.array([-0.1, -0.0]))[0] == 0
    assert formats.e2m1_encode(np.array([-0.1, -0.0]))[1] == 0


def test_e2m1_nearest_everywhere(rng):
    t = rng.uniform(-7, 7, 20000)
    got = formats.e2m1_decode(formats.e2m1_encode(t))
    grid = np.concatenate([-formats.E2M1_MAG[::-1], formats.E2M1_MAG])
    best = np.abs(np.clip(t, -6, 6)[:, None] - grid[None, :]).min(axis=1)
    assert np.allclose(np.abs(np.clip(t, -6, 6) - got), best)
