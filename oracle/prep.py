"""Offline setup of one layer (oracle): smoothing, truncated SVD, residual.

Practice page "sota-314", section "Do this": smooth the activation outliers
into the weight; take the SVD of the smoothed weight W_hat, keep the top r
singular directions in 16 bits, and quantize only the residual
R = W_hat - L1 L2.  Reading note "note-257", section "Key results": the split
puts the singular values into the first factor, L1 = U Sigma[:, :r],
L2 = V[:r, :] (rows of V^T); Eckart-Young makes this the optimal rank-r
reduction of ||W_hat||_F.

Readings where the pages are silent:
  * smoothing factor lambda_j = sqrt(max_i |X_ij| / max_n |W_jn|) (migration
    strength 1/2), in fp32, from the layer's own calibration activations;
    lambda_j = 1 when either maximum is 0;
  * X_hat = fp16_rne( fp32(X) / lambda ) (fp32 IEEE division, then one rounding
    to fp16); W_hat = lambda * W in float64 (exact);
  * SVD in float64 (LAPACK); L1 and L2 stored as fp16; the residual is taken
    against the stored fp16 factors, R = W_hat - f64(L1) f64(L2), kept as fp32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def smoothing_factors(x_cal: np.ndarray, w: np.ndarray) -> np.ndarray:
    """lambda [K] fp32 from calibration activations [M, K] and weight [K, N]."""
    mx = np.abs(np.asarray(x_cal).astype(np.float32)).max(axis=0)
    mw = np.abs(np.asarray(w).astype(np.float32)).max(axis=1)
    ok = (mx > 0) & (mw > 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lam = np.sqrt(np.where(ok, mx / np.where(ok, mw, 1), 1).astype(np.float32)).astype(np.float32)
    return np.where(ok, lam, np.float32(1.0)).astype(np.float32)


def smooth_activations(x: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """X_hat = fp16_rne(fp32(x) / lambda)."""
    return (np.asarray(x).astype(np.float32) / lam.astype(np.float32)).astype(np.float32).astype(np.float16)


def smooth_weight(w: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """W_hat = lambda * W in float64."""
    return lam.astype(np.float64)[:, None] * np.asarray(w).astype(np.float64)


def low_rank(w_hat: np.ndarray, r: int, svd=None):
    """Truncated SVD split.  Returns (L1 fp16 [K, r], L2 fp16 [r, N], R fp32 [K, N], sigma float64).

    `svd` may pass in np.linalg.svd(w_hat, full_matrices=False) when several ranks
    are split off the same smoothed weight."""
    u, sig, vt = np.linalg.svd(w_hat, full_matrices=False) if svd is None else svd
    K, N = w_hat.shape
    if r == 0:
        l1 = np.zeros((K, 0), np.float16)
        l2 = np.zeros((0, N), np.float16)
        return l1, l2, w_hat.astype(np.float32), sig
    l1 = (u[:, :r] * sig[:r]).astype(np.float16)
    l2 = vt[:r, :].astype(np.float16)
    res = w_hat - l1.astype(np.float64) @ l2.astype(np.float64)
    return l1, l2, res.astype(np.float32), sig


@dataclass
class PreparedLayer:
    lam: np.ndarray      # fp32 [K]
    x_hat: np.ndarray    # fp16 [M, K]
    l1: np.ndarray       # fp16 [K, r]
    l2: np.ndarray       # fp16 [r, N]
    res: np.ndarray      # fp32 [K, N]  (R = W_hat - L1 L2)
    bias: np.ndarray     # fp16 [N]
    sigma: np.ndarray    # float64, singular values of W_hat


def prepare_layer(x: np.ndarray, w: np.ndarray, b: np.ndarray, r: int, x_cal: np.ndarray = None,
                  svd=None) -> PreparedLayer:
    """Offline setup of one linear: smoothing from x_cal (default x), SVD split of W_hat."""
    lam = smoothing_factors(x if x_cal is None else x_cal, w)
    x_hat = smooth_activations(x, lam)
    w_hat = smooth_weight(w, lam)
    l1, l2, res, sig = low_rank(w_hat, r, svd)
    return PreparedLayer(lam, x_hat, l1, l2, res, np.asarray(b, np.float16), sig)


def lora_branch(l1: np.ndarray, l2: np.ndarray, lam: np.ndarray, a: np.ndarray, b: np.ndarray,
                scale: float = 1.0):
    """A LoRA adapter carried by the 16-bit branch (practice page "sota-314", section "Known
    implementations": the authors' engine attaches existing adapters and leaves the
    quantized weights as they are).

    The adapted layer is X (W + scale A B) with A [K, ra], B [ra, N].  In smoothed coordinates
    X = X_hat diag(lambda), so X A B = X_hat (diag(lambda) A) B and the adapter joins the
    branch:  L1' = [L1, fp16(diag(lambda) A)],  L2' = [L2; fp16(scale B)]  (products in
    float64, one rounding to fp16 each), zero-padded to a rank that is a multiple of 16 (zero
    columns / rows add exactly 0).  The residual R and its codes are unchanged.
    Returns (L1' fp16 [K, r'], L2' fp16 [r', N])."""
    K, ra = a.shape
    la = (lam.astype(np.float64)[:, None] * np.asarray(a, np.float64)).astype(np.float16)
    lb = (float(scale) * np.asarray(b, np.float64)).astype(np.float16)
    r = l1.shape[1] + ra
    pad = (-r) % 16
    l1p = np.concatenate([np.asarray(l1, np.float16), la, np.zeros((K, pad), np.float16)], axis=1)
    l2p = np.concatenate([np.asarray(l2, np.float16), lb, np.zeros((pad, lb.shape[1]), np.float16)], axis=0)
    return l1p, l2p
