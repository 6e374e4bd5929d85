"""Test-side construction of prepared layers and oracle references.

The seeded raw layers come from synth; the offline setup (smoothing, SVD,
residual) and every expected value come from the CPU oracle.  Results are
cached per process because the full-size SVDs take seconds.
"""
from __future__ import annotations

import functools
import time

import numpy as np

import oracle
from synth import CONFIGS, draw_layer, fc2_calibration_input, LayerShape

FMT_QMAX = {"int4": 7, "int8": 127}


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@functools.lru_cache(maxsize=None)
def raw_layer(name: str):
    """Raw fp16 layer for a config layer name (c0, c1_qkv, c2_fc1, c2_fc2)."""
    shapes = {s.name: s for v in CONFIGS.values() for s in v}
    if name == "c2_fc2":
        fc1 = raw_layer("c2_fc1")
        s = shapes["c2_fc2"]
        L = draw_layer(LayerShape("c2_fc2", s.M, s.K, s.N, s.r, s.fmt, s.seed, s.planted_rank))
        L.x = fc2_calibration_input(fc1)
        return L
    return draw_layer(shapes[name])


@functools.lru_cache(maxsize=None)
def _svd(name: str):
    L = raw_layer(name)
    lam = oracle.prep.smoothing_factors(L.x, L.w)
    log(f"oracle SVD of the smoothed weight of {name} {L.w.shape}")
    return np.linalg.svd(oracle.prep.smooth_weight(L.w, lam), full_matrices=False)


@functools.lru_cache(maxsize=None)
def prepared(name: str, r: int):
    log(f"oracle offline setup for {name} r={r}")
    L = raw_layer(name)
    return oracle.prep.prepare_layer(L.x, L.w, L.b, r, svd=_svd(name))


def quantize(v, fmt):
    q, s, stored = oracle.quant.quantize(v, fmt)
    return q, s, stored


_REF = {}


def reference(P, fmt, x_hat=None):
    """Oracle codes/scales/T/Y for prepared layer P (optionally another smoothed input).  On
    the layer's own input the result is kept per (layer, format) for the process."""
    if x_hat is None:
        key = (id(P), fmt)
        if key not in _REF:
            _REF[key] = _reference(P, fmt, P.x_hat)
        return _REF[key]
    return _reference(P, fmt, x_hat)


def _reference(P, fmt, x_hat):
    xq, xs, xst = quantize(x_hat, fmt)
    wq, ws, wst = quantize(P.res.T, fmt)
    t = oracle.forward.down_projection(x_hat, P.l1)
    y = oracle.forward.linear(xq, xs, t, wq, ws, P.l2, P.bias, fmt)
    return dict(xq=xq, xs=xs, xstored=xst, wq=wq, ws=ws, wstored=wst, t=t, y=y)


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb else 1.0))


def fp16_ulp_diff(a, b):
    """Max distance in fp16 units in the last place (finite inputs)."""
    def key(x):
        u = np.asarray(x, np.float16).view(np.uint16).astype(np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return int(np.max(np.abs(key(a) - key(b)))) if np.size(a) else 0


def ulp16(v):
    """fp16 unit in the last place at |v| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def within_sum_bound(got, ref, abs_sum, n_terms, extra=0.0):
    """Elementwise check for an fp16 result that is one rounding of a sum of n_terms
    (already exact or exactly-scaled) terms accumulated in fp32 in any order:
        |got - ref| <= ulp16(ref) + 2 n_terms 2^-24 sum|terms| + extra.
    The first term covers the two final roundings, the second fp32 reassociation;
    `extra` bounds differences in the inputs of the sum (e.g. an fp16 intermediate
    that each side rounded from its own accumulation)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = ulp16(np.maximum(np.abs(ref), np.abs(got))) + 2.0 * n_terms * 2.0 ** -24 * abs_sum + extra
    return bool(np.all(np.abs(got - ref) <= bound)), float(np.max(np.abs(got - ref) - bound, initial=-np.inf))


def gemm_terms(fmt, K, r):
    """Terms of the fp32 sum behind one output of Kernel B, for within_sum_bound: per-group
    partials P_g (exact) times sx sw for the INT formats; for FP4 the kernel multiplies the
    exactly dequantized values and sums all K products directly (the same exact terms,
    regrouped), so its fp32 sum has K terms; MXFP4's block-scaled matrix instruction forms
    the same exact products, counted the same way.  Plus r branch terms, the bias and the final
    rounding."""
    return (K if fmt in ("fp4", "mxfp4") else K // 64) + r + 2


def w4a16_bound_terms(x, q, s, bias):
    """(abs_sum, n_terms, extra) for within_sum_bound on the W4A16 control.  The
    kernel rounds each dequantized weight q s to fp16 once before its fp16
    matrix multiply (the usual weight-only arithmetic), while the oracle keeps
    q s exact: |fp16(w) - w| <= 2^-11 |w| + 2^-25 (the second term for fp16
    subnormals), so the inputs of the sum differ by at most
    2^-11 sum|x||w| + 2^-25 sum|x|."""
    xa = np.abs(np.asarray(x, np.float64))
    wa = np.abs(oracle.quant.dequantize(q, s, "int4"))
    xw = xa @ wa.T
    absum = xw * (1.0 + 2.0 ** -11) + 2.0 ** -25 * xa.sum(axis=1, keepdims=True)
    if bias is not None:
        absum = absum + np.abs(np.asarray(bias, np.float64))[None, :]
    extra = 2.0 ** -11 * xw + 2.0 ** -25 * xa.sum(axis=1, keepdims=True)
    return absum, xa.shape[1] + 2, extra


def linear_abs_sum(xq, xs, t, wq, ws, l2, bias, fmt):
    """sum |terms| of Y = deq(xq) deq(wq)^T + T L2 + b, elementwise (float64)."""
    xd = np.abs(oracle.quant.dequantize(xq, xs, fmt))
    wd = np.abs(oracle.quant.dequantize(wq, ws, fmt))
    s = xd @ wd.T
    if l2 is not None and l2.shape[0]:
        s += np.abs(t.astype(np.float64)) @ np.abs(l2.astype(np.float64))
    if bias is not None:
        s += np.abs(bias.astype(np.float64))[None, :]
    return s


def branch_slack(x_hat, l1, t_ref, l2):
    """Bound on |(T_gpu - T_ref) L2| when each side rounds its own T = fp16(X_hat L1):
    |T_gpu - T_ref| <= ulp16(T) + 2 K 2^-24 (|X_hat| |L1|) elementwise (the bound the
    T check enforces), propagated through |L2|."""
    K = x_hat.shape[1]
    sx = np.abs(x_hat.astype(np.float64)) @ np.abs(l1.astype(np.float64))
    dt = ulp16(t_ref) + 2.0 * K * 2.0 ** -24 * sx
    return dt @ np.abs(l2.astype(np.float64))
