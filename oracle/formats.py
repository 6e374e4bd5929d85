"""Number formats used by the layer, written from their definitions.

fp16   : IEEE binary16; conversions round to nearest, ties to even (numpy's cast).
E4M3FN : OCP 8-bit float, 1 sign, 4 exponent (bias 7), 3 mantissa bits, no
         infinities, max finite 448, S.1111.111 is NaN.  Used for the FP4
         variant's group scales (the pages give "FP8 scales" for NVFP4).
E2M1   : 4-bit float, 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
         {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Used for the FP4 variant's codes.
"""
from __future__ import annotations

import numpy as np

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E4M3_MAX = 448.0


def to_fp16(x) -> np.ndarray:
    """Round to fp16, nearest-even (IEEE), keeping subnormals."""
    return np.asarray(x).astype(np.float16)


def e4m3_decode(b) -> np.ndarray:
    """E4M3FN byte(s) -> float64 (NaN for S.1111.111)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    sub = m / 8.0 * 2.0 ** (1 - 7)
    nor = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    v = np.where(e == 0, sub, nor) * s
    return np.where((e == 15) & (m == 7), np.nan, v)


def _all_e4m3_finite_nonneg():
    codes = np.arange(0, 0x7F, dtype=np.uint8)        # 0x00 .. 0x7E (0x7F is NaN)
    return codes, e4m3_decode(codes)


def e4m3_encode_rne_sat(x) -> np.ndarray:
    """float32/64 -> E4M3FN byte, round to nearest (ties to the even code), saturating at +-448.

    The value grid is enumerated from the format definition; the nearest grid
    point wins, and on an exact tie the code with an even mantissa (equivalently
    an even code, since codes are ordered like values) is taken.  Magnitudes
    above 448 saturate to 448.  Negative values get the sign bit; -0 encodes as
    +0.  Non-finite inputs are not expected (scales are absmax / 6 of finite data).
    """
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _all_e4m3_finite_nonneg()
    a = np.minimum(np.abs(x), E4M3_MAX)
    # index of the largest grid value <= a
    lo = np.searchsorted(vals, a, side="right") - 1
    lo = np.clip(lo, 0, len(vals) - 1)
    hi = np.minimum(lo + 1, len(vals) - 1)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (codes[hi] % 2 == 0) & (hi != lo))
    c = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    neg = (x < 0) & (c != 0)
    return np.where(neg, c | 0x80, c).astype(np.uint8)


def e2m1_decode(nib) -> np.ndarray:
    """4-bit E2M1 code (sign<<3 | magnitude index) -> float64."""
    nib = np.asarray(nib, dtype=np.int64)
    v = E2M1_MAG[nib & 7]
    return np.where(nib & 8, -v, v)


def e2m1_encode(t) -> np.ndarray:
    """Nearest E2M1 value to t (|t| clamped to 6), ties to the even mantissa; -0 -> +0.

    Tie points and their winners: 0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2,
    3.5->4, 5->4 (the neighbour whose mantissa bit is 0).
    """
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(t), 6.0)
    d = np.abs(a[..., None] - E2M1_MAG)                 # distance to each magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # among tied candidates prefer an even mantissa bit; mantissa bit of index i is i & 1 for i >= 2,
    # and index 1 (0.5, subnormal) has mantissa bit 1, index 0 has 0.
    even = (np.arange(8) & 1) == 0
    pref = cand & even
    idx = np.where(pref.any(axis=-1), np.argmax(pref, axis=-1), np.argmax(cand, axis=-1))
    neg = (t < 0) & (idx != 0)
    return (idx | np.where(neg, 8, 0)).astype(np.uint8)


def e8m0_decode(b) -> np.ndarray:
    """E8M0 scale byte (OCP Microscaling Formats v1.0: an 8-bit biased exponent, no sign or
    mantissa) -> 2^(b - 127) as float64; 255 (NaN) is never produced here."""
    return np.ldexp(1.0, np.asarray(b, dtype=np.int64) - 127)
