"""GPTQ rounding of the residual (oracle).

Practice page "sota-314", section "Do this": the authors' pipeline rounds the residual with
GPTQ instead of to nearest, and reports better quality for it in most settings; the default
here stays round-to-nearest (codes as a pure function of the weights).  GPTQ (Frantar, Ashkboos,
Hoefler, Alistarh 2022, "GPTQ: Accurate Post-Training Quantization for Generative
Pre-trained Transformers", Algorithm 1) rounds the weight one input channel (column of K) at
a time and spreads each column's rounding error over the channels not yet rounded, weighted
by the inverse Hessian of the layer's squared output error, H = 2 X^T X over calibration
activations X (here the smoothed X_hat the residual multiplies).

Plain form written from the algorithm's steps (no lazy batching, which only regroups the
same updates), in float64, per output column row w of R^T [N, K]:
  * H <- H + damp * mean(diag H) * I; a channel with H_jj = 0 (never active) gets H_jj = 1
    and its weights set to 0;
  * U = the upper Cholesky factor of H^-1 (H^-1 = U^T U);
  * for j = 0 .. K-1: at the first channel of each group of G, the group's scale is taken
    from the current (already updated) weights of that group with the round-to-nearest
    rule; q_j = the round-to-nearest code of w_j against that scale;
    d = (w_j - q_j s) / U_jj;  w_{j+1..} -= d * U_{j, j+1..}.
Codes and scales use exactly the element rule of quant.quantize_int (fp32 value, fp16
scale = fp16_rne(fp32(absmax) / qmax), RNE quotient, clamp); with H a multiple of the
identity the updates vanish and GPTQ gives the round-to-nearest codes.
"""
from __future__ import annotations

import numpy as np

from .quant import INT4_QMAX, INT8_QMAX


def _scale(a32: np.ndarray, qmax: int) -> np.ndarray:
    return (a32 / np.float32(qmax)).astype(np.float32).astype(np.float16)


def _codes(col32: np.ndarray, s: np.ndarray, qmax: int) -> np.ndarray:
    sf = s.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = col32 / sf
    t = np.where(sf == 0, 0.0, t)
    return np.clip(np.rint(t), -qmax, qmax).astype(np.int8)


def hessian(x_cal: np.ndarray) -> np.ndarray:
    """H = 2 X^T X in float64 over calibration activations X [M, K]."""
    x = np.asarray(x_cal, np.float64)
    return 2.0 * x.T @ x


def gptq(r_t: np.ndarray, h: np.ndarray, fmt: str, damp: float = 0.01, G: int = 64):
    """GPTQ codes and scales of R^T [N, K] (rows = output columns) for an INT format.
    Returns (codes int8 [N, K], scales fp16 [N, K/G])."""
    qmax = {"int4": INT4_QMAX, "int4_e2m3": INT4_QMAX, "int8": INT8_QMAX}[fmt]
    w = np.array(r_t, dtype=np.float64)
    N, K = w.shape
    h = np.array(h, dtype=np.float64)
    dead = np.diag(h) == 0
    h[dead, dead] = 1.0
    w[:, dead] = 0.0
    h += damp * np.mean(np.diag(h)) * np.eye(K)
    u = np.linalg.cholesky(np.linalg.inv(h)).T          # upper: H^-1 = U^T U
    codes = np.zeros((N, K), np.int8)
    scales = np.zeros((N, K // G), np.float16)
    for j in range(K):
        g = j // G
        if j % G == 0:
            blk = w[:, j:j + G].astype(np.float32)
            scales[:, g] = _scale(np.abs(blk).max(axis=1), qmax)
        q = _codes(w[:, j].astype(np.float32), scales[:, g], qmax)
        codes[:, j] = q
        d = (w[:, j] - q.astype(np.float64) * scales[:, g].astype(np.float64)) / u[j, j]
        w[:, j + 1:] -= d[:, None] * u[j, j + 1:][None, :]
    return codes, scales
