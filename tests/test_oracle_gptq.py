"""Pins of the oracle's GPTQ: it reduces to round-to-nearest when H is a multiple of the
identity, a two-channel case reproduces the optimal-brain-surgeon update in closed form, and
on correlated calibration data it lowers the layer's output error below round-to-nearest's.
CPU only."""
import numpy as np
import pytest

from oracle import gptq, quant


@pytest.mark.parametrize("fmt,qmax", [("int4", 7), ("int8", 127)])
def test_gptq_with_identity_hessian_is_round_to_nearest(fmt, qmax):
    g = np.random.default_rng(3)
    r_t = (g.standard_normal((24, 128)) * 0.05).astype(np.float32)
    codes, scales = gptq.gptq(r_t, 3.0 * np.eye(128), fmt)
    q, s = quant.quantize_int(r_t, qmax, 64)
    assert np.array_equal(codes, q) and np.array_equal(scales.view(np.uint16), s.view(np.uint16))


def test_gptq_two_channels_obs_update_closed_form():
    # one group of two channels: after rounding channel 0 to q0 s, the remaining weight moves
    # by d0 * (-[H^-1]_01 / [H^-1]_00) = d0 * b / c for H = [[a, b], [b, c]] (d0 = w0 - q0 s),
    # then is rounded against the same scale
    # (w1 is the group's maximum, so the scale is 0.7 / 7 and w0 / s = 3.49 leaves d0 = 0.049;
    # b / c = -2 pulls w1 from 7.0 s to 6.02 s)
    a, b, c = 5.0, -2.4, 1.2
    w0, w1 = 0.349, 0.7
    h = np.array([[a, b], [b, c]])
    codes, scales = gptq.gptq(np.array([[w0, w1]], np.float32), h, "int4", damp=0.0, G=2)
    s = np.float64(np.float16(np.float32(0.7) / np.float32(7)))
    q0 = np.clip(np.rint(np.float32(w0) / np.float32(s)), -7, 7)
    d0 = np.float64(np.float32(w0)) - q0 * s
    w1p = np.float64(np.float32(w1)) + d0 * b / c
    q1 = np.clip(np.rint(np.float32(w1p) / np.float32(s)), -7, 7)
    assert float(scales[0, 0]) == s
    assert list(codes[0]) == [q0, q1]
    assert q1 != np.clip(np.rint(np.float32(w1) / np.float32(s)), -7, 7)   # the update changed the code


def test_gptq_lowers_output_error_on_correlated_inputs():
    g = np.random.default_rng(4)
    M, K, N = 512, 128, 48
    mix = g.standard_normal((K, K)) * 0.3 + np.eye(K)
    x = (g.standard_normal((M, K)) @ mix).astype(np.float16)          # correlated channels
    r_t = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    codes, scales = gptq.gptq(r_t, gptq.hessian(x), "int4")
    q_rtn, s_rtn = quant.quantize_int(r_t, 7, 64)
    xd = x.astype(np.float64)
    err_gptq = np.linalg.norm(xd @ (r_t - quant.dequant_int(codes, scales)).T)
    err_rtn = np.linalg.norm(xd @ (r_t - quant.dequant_int(q_rtn, s_rtn)).T)
    assert err_gptq < 0.8 * err_rtn
    assert np.abs(codes).max() <= 7
