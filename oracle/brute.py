"""Brute force of the layer for tiny shapes (oracle cross-check).

Plain Python loops over the per-group integer form
    Y[m, n] = fp16( sum_g s_x[m, g] s_w[n, g] P_g[m, n] + sum_j T[m, j] L2[j, n] + b[n] ),
    P_g[m, n] = sum_{k in g} q_x[m, k] q_w[n, k]   (exact Python integers),
with T[m, j] = fp16( sum_k X_hat[m, k] L1[k, j] ) accumulated with math.fsum.
Independent of forward.py: no matrix products, no shared helpers beyond the
fp16 cast.  INT formats only (the FP4 form is pinned by its own tables).
"""
from __future__ import annotations

import math

import numpy as np


def _f16(x: float) -> float:
    return float(np.float16(x))


def down_projection(x_hat, l1):
    M, K = x_hat.shape
    r = l1.shape[1]
    t = np.zeros((M, r), np.float16)
    for m in range(M):
        for j in range(r):
            t[m, j] = _f16(math.fsum(float(x_hat[m, k]) * float(l1[k, j]) for k in range(K)))
    return t


def linear(xq, xs, t, wq, ws, l2, bias, G=64):
    """xq [M,K] int codes, xs fp16 [M,K/G]; wq [N,K] int codes, ws fp16 [N,K/G]; t fp16 [M,r]; l2 fp16 [r,N]."""
    M, K = xq.shape
    N = wq.shape[0]
    r = 0 if l2 is None else l2.shape[0]
    y = np.zeros((M, N), np.float16)
    for m in range(M):
        for n in range(N):
            terms = []
            for g in range(K // G):
                p = 0
                for k in range(g * G, (g + 1) * G):
                    p += int(xq[m, k]) * int(wq[n, k])
                terms.append(float(xs[m, g]) * float(ws[n, g]) * p)
            for j in range(r):
                terms.append(float(t[m, j]) * float(l2[j, n]))
            if bias is not None:
                terms.append(float(bias[n]))
            y[m, n] = _f16(math.fsum(terms))
    return y
