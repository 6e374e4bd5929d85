"""Pins of the oracle's forward pass.

* exact grid: X_hat and R on the int4 grid (q 2^-4, a +-7 in every group), no
  branch, no bias -> Y equals fp16 of the exact integer product, bit for bit;
* brute force: independent float64 loops of the per-group integer form;
* the output-error bound by magnitudes and rounding errors (reading note
  "note-257", section "Key results", first proposition; the inequality below is
  its triangle-inequality form, the pages do not print it);
* GELU(tanh) vs torch; W4A16 vs loops;
* the method's ordering on a synthetic outlier layer: smoothing + low-rank +
  4-bit residual beats plain 4-bit quantization of both operands (practice
  page "sota-314", section "Do this").
"""
import numpy as np
import pytest
import torch

from oracle import quant, prep, forward, brute
from synth import draw_layer, LayerShape


def _grid(rng, rows, K):
    q = rng.integers(-7, 8, (rows, K))
    for g in range(K // 64):
        q[np.arange(rows), g * 64 + rng.integers(0, 64, rows)] = rng.choice([-7, 7], rows)
    return q


@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (17, 128, 48), (64, 256, 32)])
def test_exact_grid_bit_for_bit(rng, M, K, N):
    qx, qr = _grid(rng, M, K), _grid(rng, N, K)
    x_hat = (qx * 2.0 ** -4).astype(np.float16)
    r_t = (qr * 2.0 ** -4).astype(np.float32)          # R^T [N, K]
    xq, xs = quant.quantize_int(x_hat, 7, 64)
    wq, ws = quant.quantize_int(r_t, 7, 64)
    assert np.array_equal(xq, qx) and np.array_equal(wq, qr)
    y = forward.linear(xq, xs, np.zeros((M, 0), np.float16), wq, ws, np.zeros((0, N), np.float16), None, "int4")
    exact = (qx.astype(object) @ qr.T.astype(object))    # python ints
    ref = np.array([[float(v) * 2.0 ** -8 for v in row] for row in exact]).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("M,K,N,r", [(1, 64, 16, 0), (3, 128, 32, 16), (17, 64, 48, 32), (5, 128, 16, 32)])
def test_brute_force_int4(M, K, N, r):
    g = np.random.default_rng(M * 1000 + K + N + r)
    x_hat = (g.standard_normal((M, K)) * 0.7).astype(np.float16)
    r_t = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    l1 = (g.standard_normal((K, r)) * 0.2).astype(np.float16)
    l2 = (g.standard_normal((r, N)) * 0.2).astype(np.float16)
    b = (g.standard_normal(N) * 0.01).astype(np.float16)
    xq, xs = quant.quantize_int(x_hat, 7, 64)
    wq, ws = quant.quantize_int(r_t, 7, 64)
    t = forward.down_projection(x_hat, l1)
    assert np.array_equal(t.view(np.uint16), brute.down_projection(x_hat, l1).view(np.uint16))
    y = forward.linear(xq, xs, t, wq, ws, l2, b, "int4")
    yb = brute.linear(xq, xs, t, wq, ws, l2, b)
    assert np.array_equal(y.view(np.uint16), yb.view(np.uint16))


def test_brute_force_int8():
    g = np.random.default_rng(5)
    M, K, N, r = 4, 128, 16, 16
    x_hat = (g.standard_normal((M, K))).astype(np.float16)
    r_t = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    l1 = (g.standard_normal((K, r)) * 0.2).astype(np.float16)
    l2 = (g.standard_normal((r, N)) * 0.2).astype(np.float16)
    xq, xs = quant.quantize_int(x_hat, 127, 64)
    wq, ws = quant.quantize_int(r_t, 127, 64)
    t = forward.down_projection(x_hat, l1)
    y = forward.linear(xq, xs, t, wq, ws, l2, None, "int8")
    assert np.array_equal(y.view(np.uint16), brute.linear(xq, xs, t, wq, ws, l2, None).view(np.uint16))


def test_fp4_gemm_against_loops():
    g = np.random.default_rng(9)
    M, K, N = 3, 64, 8
    x = g.standard_normal((M, K)).astype(np.float32)
    w = g.standard_normal((N, K)).astype(np.float32)
    xq, xs = quant.quantize_fp4(x, 16)
    wq, ws = quant.quantize_fp4(w, 16)
    z = forward.lowbit_gemm(xq, xs, wq, ws, "fp4")
    from oracle.formats import e2m1_decode, e4m3_decode
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(e2m1_decode(xq[m, k])) * float(e4m3_decode(xs[m, k // 16])) * \
                       float(e2m1_decode(wq[n, k])) * float(e4m3_decode(ws[n, k // 16]))
            assert np.isclose(z[m, n], acc, rtol=1e-12, atol=1e-12)


def test_output_error_bound_by_magnitudes(rng):
    x = rng.standard_normal((32, 256))
    w = rng.standard_normal((256, 48)) * 0.1
    xq, xs = quant.quantize_int(x.astype(np.float32), 7, 64)
    wq, ws = quant.quantize_int(w.T.astype(np.float32), 7, 64)
    qx = quant.dequant_int(xq, xs)
    qw = quant.dequant_int(wq, ws).T
    lhs = np.linalg.norm(x @ w - qx @ qw)
    ex, ew = np.linalg.norm(x - qx), np.linalg.norm(w - qw)
    rhs = np.linalg.norm(x) * ew + ex * (np.linalg.norm(w) + ew)
    assert lhs <= rhs


def test_gelu_matches_torch(rng):
    y = (rng.standard_normal(20000) * 3).astype(np.float64)
    ref = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.allclose(forward.gelu_tanh(y), ref, rtol=1e-14, atol=1e-15)


def test_gelu_smooth_rounding(rng):
    y = (rng.standard_normal((8, 32)) * 2).astype(np.float16)
    lam = (rng.uniform(0.5, 4, 32)).astype(np.float32)
    out = forward.gelu_smooth(y, lam)
    ref = torch.nn.functional.gelu(torch.from_numpy(y.astype(np.float64)), approximate="tanh").numpy() / lam.astype(np.float64)
    assert np.array_equal(out, ref.astype(np.float16))


def test_w4a16_against_loops():
    g = np.random.default_rng(4)
    M, K, N = 3, 128, 8
    x = g.standard_normal((M, K)).astype(np.float16)
    w_t = (g.standard_normal((N, K)) * 0.05).astype(np.float16)
    b = (g.standard_normal(N) * 0.01).astype(np.float16)
    wq, ws = quant.quantize_int(w_t, 7, 64)
    y = forward.w4a16(x, wq, ws, b)
    import math
    for m in range(M):
        for n in range(N):
            acc = math.fsum([float(x[m, k]) * int(wq[n, k]) * float(ws[n, k // 64]) for k in range(K)] + [float(b[n])])
            assert y[m, n] == np.float16(acc)


def test_method_beats_plain_w4a4_on_outlier_layer():
    L = draw_layer(LayerShape("t", 256, 512, 256, 32, "int4", 1234, 8))
    ref = L.x.astype(np.float64) @ L.w.astype(np.float64) + L.b.astype(np.float64)

    def err(y):
        return np.linalg.norm(y.astype(np.float64) - ref) / np.linalg.norm(ref)
    # plain W4A4: quantize X and W directly
    xq, xs = quant.quantize_int(L.x, 7, 64)
    wq, ws = quant.quantize_int(L.w.T.astype(np.float32), 7, 64)
    naive = forward.linear(xq, xs, np.zeros((256, 0), np.float16), wq, ws, np.zeros((0, 256), np.float16), L.b, "int4")
    # SVDQuant: smoothing + rank-32 branch + 4-bit residual
    P = prep.prepare_layer(L.x, L.w, L.b, 32)
    xq, xs = quant.quantize_int(P.x_hat, 7, 64)
    wq, ws = quant.quantize_int(P.res.T, 7, 64)
    t = forward.down_projection(P.x_hat, P.l1)
    svdq = forward.linear(xq, xs, t, wq, ws, P.l2, P.bias, "int4")
    assert err(svdq) < 0.5 * err(naive)
