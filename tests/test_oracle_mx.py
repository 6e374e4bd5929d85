"""Pins of the oracle's MXFP4 quantizer (E2M1 codes, group 32, E8M0 scales; OCP Microscaling
Formats v1.0): groups worked by hand from the definition, exact round trips on the grid, the
error bound, and a brute-force nearest-code search.  CPU only."""
import numpy as np
import pytest

from oracle import quant
from oracle.formats import E2M1_MAG


def group(values, fill=0.0):
    v = np.full(32, fill, np.float64)
    v[:len(values)] = values
    return v[None, :]


# (group's leading values, expected E8M0 byte, expected leading codes), each worked by hand:
# e = floor(log2 max|v|) - 2, byte = e + 127, code = nearest E2M1 to v / 2^e (ties to the even
# mantissa, saturating at 6; sign<<3 | magnitude index over 0, .5, 1, 1.5, 2, 3, 4, 6)
HAND = [
    ([6.0, -3.0, 1.5, 0.5], 127, [7, 13, 3, 1]),              # max 6: e = 2 - 2 = 0, X = 1
    ([7.0, 1.0, -7.0], 127, [7, 2, 15]),                      # max 7: e = 0, 7 saturates to 6
    ([8.0, 2.5, -0.75], 128, [6, 2, 9]),                      # max 8: e = 1, X = 2: 4, 1.25 -> 1 (tie), -0.375 -> -0.5
    ([2.0 ** -24, -2.0 ** -25], 101, [6, 12]),                # fp16 subnormals: e = -24 - 2, v / X = 4, -2
    ([0.1, 0.05], 121, [7, 5]),                               # max 0.1: floor(log2 0.1) = -4, e = -6: 6.4 -> 6, 3.2 -> 3
    ([3e38, 1e38], 252, [7, 4]),                              # fp32 near max: e = 127 - 2: 7.05 -> 6, 2.35 -> 2
    ([1e-40], 0, [0]),                                        # fp32 subnormal: e clamps to -127, v / X = 0.017 -> 0
    ([0.0, -0.0], 0, [0, 0]),                                 # an all-zero group: byte 0, codes +0
]


@pytest.mark.parametrize("values,byte,codes", HAND)
def test_mx_hand_worked_groups(values, byte, codes):
    q, s = quant.quantize_mx(group(values).astype(np.float32))
    assert int(s[0, 0]) == byte
    assert list(q[0, :len(codes)]) == codes


def test_mx_hand_case_near_fp32_max_in_detail():
    # 3e38 = 1.763 * 2^127 -> e = 125; 3e38 / 2^125 = 7.05 (saturates to 6, index 7);
    # 1e38 / 2^125 = 2.35, between 2 (index 4) and 3 (index 5), nearer 2
    q, s = quant.quantize_mx(group([3e38, 1e38]).astype(np.float32))
    assert int(s[0, 0]) == 252 and list(q[0, :2]) == [7, 4]


def test_mx_grid_values_round_trip_exactly():
    g = np.random.default_rng(1)
    rows, K = 16, 128
    k = g.integers(-20, 20, (rows, K // 32))
    idx = g.integers(0, 16, (rows, K))
    idx[:, ::32] = 7                                   # each group's largest magnitude is 6 * 2^k
    v = (np.where(idx & 8, -1, 1) * E2M1_MAG[idx & 7]).reshape(rows, -1, 32) * np.ldexp(1.0, k)[..., None]
    v = v.reshape(rows, K).astype(np.float32)
    q, s = quant.quantize_mx(v)
    assert np.array_equal(quant.dequant_mx(q, s), v.astype(np.float64))
    assert np.array_equal(s.astype(np.int64), k + 127)


def test_mx_error_bound_and_brute_force_nearest_code():
    g = np.random.default_rng(2)
    v = (g.standard_normal((64, 256)) * 10.0 ** g.integers(-3, 3, (64, 1))).astype(np.float32)
    q, s = quant.quantize_mx(v)
    X = np.ldexp(1.0, s.astype(np.int64) - 127)
    Xe = np.repeat(X, 32, axis=1)
    d = quant.dequant_mx(q, s)
    t = v.astype(np.float64) / Xe
    assert np.all(np.abs(d - v) <= np.where(np.abs(t) > 6, 2.0, 1.0) * Xe)   # half-spacing <= 1 X; saturation < 2 X
    # brute force: the code of every element is the nearest of the 16 E2M1 values to v / X
    # (continuous random data has no ties), the largest magnitude clamped to 6
    cand = np.concatenate([E2M1_MAG, -E2M1_MAG])
    best = cand[np.argmin(np.abs(t[..., None] - cand), axis=-1)]
    assert np.array_equal(quant.dequant_mx(q, s) / Xe, best)
    # every group's largest |v| / X lies in [4, 8): the exponent rule puts it there
    a = np.abs(v.astype(np.float64)).reshape(64, -1, 32).max(axis=-1) / X
    assert np.all((a >= 4) & (a < 8))
