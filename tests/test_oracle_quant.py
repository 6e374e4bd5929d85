"""Pins of the oracle's group quantizers.

* hand-worked examples (tests/golden/quant_examples.json);
* the per-element rounding bound |v - q s| <= s/2 whenever the fp16 scale is
  normal (the magnitude bound on rounding error the method's second
  proposition rests on: reading note "note-257", section "Key results");
* exact rational arithmetic for scales and codes (definition, not numpy casts);
* exact round trip on the integer grid; ties to even; zero groups; packing.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, formats
from tests.exact import rn_fp32, rn_fp16, rn_e4m3_sat, rint_even

GOLD = os.path.join(os.path.dirname(__file__), "golden", "quant_examples.json")


def _group(vals, G):
    v = np.zeros((1, G), np.float32)
    v[0, :len(vals)] = np.array(vals, np.float32)
    return v


def test_golden_int4_examples():
    ex = json.load(open(GOLD))["int4"]
    for e in ex:
        v = _group(e["v"], 64)
        q, s = quant.quantize_int(v, 7, 64)
        assert int(s.view(np.uint16)[0, 0]) == e["scale_fp16_bits"], e["derivation"]
        assert list(q[0, :len(e["codes"])]) == e["codes"]
        assert not q[0, len(e["codes"]):].any()
        p = quant.pack_nibbles(q)
        assert list(p[0, :len(e["packed_first_bytes"])]) == e["packed_first_bytes"]


def test_golden_fp4_examples():
    ex = json.load(open(GOLD))["fp4"]
    for e in ex:
        v = _group(e["v"], 16)
        q, s = quant.quantize_fp4(v, 16)
        assert int(s[0, 0]) == e["scale_e4m3"], e["derivation"]
        assert list(q[0, :len(e["nibbles"])]) == e["nibbles"]
        p = quant.pack_nibbles(q)
        assert list(p[0, :len(e["packed_first_bytes"])]) == e["packed_first_bytes"]


def _data(rng, rows, K, kind):
    if kind == "normal":
        return rng.standard_normal((rows, K)).astype(np.float32)
    if kind == "outlier":
        x = rng.standard_normal((rows, K))
        x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 30
        return x.astype(np.float16).astype(np.float32)
    if kind == "tiny":     # pushes scales into fp16 subnormals
        return (rng.standard_normal((rows, K)) * 1e-6).astype(np.float32)
    if kind == "wide":
        return (rng.standard_normal((rows, K)) * 10.0 ** rng.integers(-3, 3, (rows, 1))).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("qmax", [7, 127])
@pytest.mark.parametrize("kind", ["normal", "outlier", "wide"])
def test_rounding_error_bound_int(rng, qmax, kind):
    v = _data(rng, 64, 512, kind)
    q, s16 = quant.quantize_int(v, qmax, 64)
    s = np.repeat(s16.astype(np.float64), 64, axis=1)
    normal = np.repeat((np.abs(s16.astype(np.float32)) >= np.float32(2.0 ** -14)), 64, axis=1)
    err = np.abs(v.astype(np.float64) - q.astype(np.float64) * s)
    assert (err[normal] <= s[normal] / 2 * (1 + 1e-6)).all()
    # the clamp is inactive where the scale is normal: the unclamped code is within range
    t = np.rint(v.astype(np.float64) / np.where(s == 0, 1, s))
    assert (np.abs(t[normal]) <= qmax).all()
    assert q.min() >= -qmax and q.max() <= qmax


def test_int4_never_minus_eight(rng):
    v = _data(rng, 128, 1024, "tiny")
    q, _ = quant.quantize_int(v, 7, 64)
    assert q.min() >= -7


@pytest.mark.parametrize("qmax,kind", [(7, "normal"), (7, "tiny"), (127, "outlier"), (7, "wide")])
def test_scales_and_codes_exact_rational(rng, qmax, kind):
    v = _data(rng, 4, 128, kind)
    q, s16 = quant.quantize_int(v, qmax, 64)
    for i in range(v.shape[0]):
        for g in range(2):
            grp = [Fraction(float(x)) for x in v[i, g * 64:(g + 1) * 64]]
            a = max(abs(x) for x in grp)
            s = rn_fp16(rn_fp32(a / qmax))
            assert Fraction(float(s16[i, g])) == s
            for k, x in enumerate(grp):
                code = 0 if s == 0 else max(-qmax, min(qmax, rint_even(rn_fp32(x / s))))
                assert int(q[i, g * 64 + k]) == code


def test_fp4_exact_rational(rng):
    v = _data(rng, 8, 64, "wide")
    q, s8 = quant.quantize_fp4(v, 16)
    for i in range(v.shape[0]):
        for g in range(4):
            grp = [Fraction(float(x)) for x in v[i, g * 16:(g + 1) * 16]]
            a = max(abs(x) for x in grp)
            s = rn_e4m3_sat(rn_fp32(a / 6))
            assert Fraction(float(formats.e4m3_decode(s8[i, g]))) == s
            for k, x in enumerate(grp):
                t = rn_fp32(x / s) if s else Fraction(0)
                # nearest E2M1 magnitude with ties to the even mantissa, computed from the grid
                mags = [Fraction(m) for m in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
                at = min(abs(t), Fraction(6))
                d = [abs(at - m) for m in mags]
                best = min(d)
                cands = [j for j in range(8) if d[j] == best]
                j = [c for c in cands if c % 2 == 0][0] if len(cands) > 1 else cands[0]
                val = -mags[j] if t < 0 else mags[j]
                assert Fraction(float(formats.e2m1_decode(q[i, g * 16 + k]))) == val


def test_fp4_error_bounds(rng):
    v = _data(rng, 64, 256, "outlier")
    q, s8 = quant.quantize_fp4(v, 16)
    s = np.repeat(formats.e4m3_decode(s8), 16, axis=1)
    deq = formats.e2m1_decode(q) * s
    t = np.abs(v.astype(np.float64)) / np.where(s == 0, 1, s)
    spacing = np.where(t < 2, 0.5, np.where(t < 4, 1.0, 2.0))
    inside = t <= 6
    err = np.abs(v - deq)
    assert (err[inside] <= (spacing * s / 2)[inside] * (1 + 1e-6)).all()
    sat = ~inside
    assert (err[sat] <= (np.abs(v) - 6 * s)[sat] * (1 + 1e-6) + 1e-30).all()


def test_exact_grid_round_trip(rng):
    # v = q * 2^-4 with |q| <= 7 and a +-7 in every group: s = 2^-4 exactly and codes come back
    rows, K = 16, 256
    q = rng.integers(-7, 8, (rows, K))
    for g in range(K // 64):
        q[:, g * 64 + rng.integers(0, 64)] = rng.choice([-7, 7], rows)
    v = (q * 2.0 ** -4).astype(np.float32)
    qq, s = quant.quantize_int(v, 7, 64)
    assert np.array_equal(qq, q)
    assert (s.astype(np.float64) == 2.0 ** -4).all()


def test_ties_go_to_even():
    # s = 1 (absmax 7): v = n + 1/2 -> even neighbour
    v = np.zeros((1, 64), np.float32)
    v[0, 0] = 7.0
    halves = [-6.5, -5.5, -4.5, -3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5]
    v[0, 1:1 + len(halves)] = halves
    q, s = quant.quantize_int(v, 7, 64)
    assert float(s[0, 0]) == 1.0
    assert list(q[0, 1:1 + len(halves)]) == [-6, -6, -4, -4, -2, -2, 0, 0, 2, 2, 4, 4, 6, 6]


def test_zero_group():
    v = np.zeros((2, 128), np.float32)
    v[1, 64:] = 1.0
    q, s = quant.quantize_int(v, 7, 64)
    assert float(s[0, 0]) == 0 and float(s[0, 1]) == 0 and float(s[1, 0]) == 0
    assert not q[0].any() and not q[1, :64].any()
    qf, sf = quant.quantize_fp4(v, 16)
    assert not qf[0].any() and not sf[0].any()


def test_packing_round_trip(rng):
    q = rng.integers(-7, 8, (5, 128)).astype(np.int8)
    p = quant.pack_nibbles(q)
    assert p.shape == (5, 64)
    assert (p[:, 0] & 0xF).tolist() == (q[:, 0] & 0xF).tolist()
    assert (p[:, 0] >> 4).tolist() == (q[:, 1] & 0xF).tolist()
    assert np.array_equal(quant.unpack_int4(p), q)
    nib = rng.integers(0, 16, (3, 32)).astype(np.uint8)
    assert np.array_equal(quant.unpack_nibbles(quant.pack_nibbles(nib)), nib)


def test_e2m3_format_has_int4_codes_and_scales(rng):
    v = rng.standard_normal((8, 128)).astype(np.float32)
    q4, s4, st4 = quant.quantize(v, "int4")
    q6, s6, st6 = quant.quantize(v, "int4_e2m3")
    assert np.array_equal(q4, q6) and np.array_equal(s4.view(np.uint16), s6.view(np.uint16))
    assert np.array_equal(st6, st4) and np.array_equal(quant.unpack_int4(st6), q4)


def _fma32(a, b, c):
    """IEEE fp32 fused multiply-add RN32(a*b + c) of float32 arrays, exactly: the product is
    exact in float64, TwoSum gives the sum as s + err exactly, and the only case where
    RN32(s) differs from RN32(s + err) is s on an fp32 midpoint with err != 0."""
    p = a.astype(np.float64) * b.astype(np.float64)
    c64 = c.astype(np.float64)
    s = p + c64
    bb = s - p
    err = (p - (s - bb)) + (c64 - bb)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    up = np.where(r64 < s, np.nextafter(r, np.float32(np.inf)), r)
    down = np.where(r64 > s, np.nextafter(r, np.float32(-np.inf)), r)
    mid = (up != down) & (s == (up.astype(np.float64) + down.astype(np.float64)) / 2)
    return np.where(mid & (err > 0), up, np.where(mid & (err < 0), down, r)).astype(np.float32)


def _fast_code(x32, s32, qmax, r_ulps=0):
    """Kernel A's code rule, simulated in IEEE fp32: r = a reciprocal of s within one ulp
    (r_ulps moves RN(1/s) by one ulp either way, as v_rcp_f32 may), t0 = RN(x r), one fma
    refinement t = fma(fma(-t0, s, x), r, t0), then clamp and round half to even."""
    with np.errstate(divide="ignore"):
        r = np.where(s32 == 0, np.float32(0), np.float32(1) / s32).astype(np.float32)
    if r_ulps:
        r = np.where(s32 == 0, r, np.nextafter(r, np.float32(np.inf * r_ulps))).astype(np.float32)
    t0 = (x32 * r).astype(np.float32)
    t = _fma32(_fma32(-t0, s32, x32), r, t0)
    return np.rint(np.clip(t, -qmax, qmax))


@pytest.mark.parametrize("qmax", [7, 127])
@pytest.mark.parametrize("r_ulps", [0, 1, -1])
def test_division_free_code_rule_matches_definition_exhaustively(qmax, r_ulps):
    """Every fp16 value against a spread of fp16 scales (normal and subnormal), with the
    reciprocal correctly rounded or one ulp off either way: the kernel's reciprocal-and-
    refinement rule gives clamp(rint(fp32(x) / s)) exactly."""
    xs = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)   # all finite >= 0
    xs = np.concatenate([xs, -xs])
    g = np.random.default_rng(qmax)
    scales = np.concatenate([
        np.arange(1, 1024, 37, dtype=np.uint16),                 # subnormal fp16 scales
        g.integers(0x0400, 0x7BFF, 120).astype(np.uint16),       # normal fp16 scales
        np.array([0x3C00, 0x3800, 0x2E66, 0x0001, 0x03FF, 0x7BFF], np.uint16),
    ]).view(np.float16).astype(np.float32)
    for s in scales:
        s32 = np.float32(s)
        ref = np.clip(np.rint((xs / s32).astype(np.float32)), -qmax, qmax)
        got = _fast_code(xs, np.full_like(xs, s32), qmax, r_ulps)
        assert np.array_equal(got, ref), float(s)
    # the zero scale gives code 0
    assert not _fast_code(xs[:100], np.zeros(100, np.float32), qmax).any()


def test_fma32_emulation():
    # the fp32 fma emulation against exact rational arithmetic on random and cancelling inputs
    from fractions import Fraction
    g = np.random.default_rng(5)
    a = g.standard_normal(3000).astype(np.float32)
    b = g.standard_normal(3000).astype(np.float32)
    c = np.where(g.random(3000) < 0.5, -(a * b).astype(np.float32), g.standard_normal(3000).astype(np.float32))
    got = _fma32(a, b, c)
    for i in range(3000):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        lo = np.float32(float(exact))                  # candidates around the exact value
        cands = [lo, np.nextafter(lo, np.float32(np.inf)), np.nextafter(lo, np.float32(-np.inf))]
        best = min(cands, key=lambda v: (abs(Fraction(float(v)) - exact), int(np.float32(v).view(np.uint32)) & 1))
        assert got[i] == best, (a[i], b[i], c[i])


@pytest.mark.parametrize("qmax", [7, 127])
def test_division_free_scale_rule_exhaustively(qmax):
    """Kernel A's scale fp16_rne(amax * RN(1/qmax)) equals fp16_rne(RN(amax / qmax)) for every
    finite fp16 absmax."""
    a = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    ref = (a / np.float32(qmax)).astype(np.float32).astype(np.float16)
    got = (a * (np.float32(1) / np.float32(qmax))).astype(np.float32).astype(np.float16)
    assert np.array_equal(ref.view(np.uint16), got.view(np.uint16))
