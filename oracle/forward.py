"""The layer's forward pass (oracle), in float64 with the rounding points the layer fixes.

Practice page "sota-314", section "Do this": the 16-bit low-rank branch runs
beside the 4-bit GEMM on the residual, Y = X_hat L1 L2 + Q(X_hat) Q(R) + b;
the fused kernels pair the down projection with quantization (same input) and
the up projection with the 4-bit GEMM's output (same output).

Rounding points (readings, the pages give only "16-bit"):
  T = fp16_rne( X_hat L1 )                    the branch's intermediate is stored in fp16
  Z = sum over groups of (q_x s_x) (q_w s_w)  the dequantized-operand GEMM (plain definition)
  Y = fp16_rne( Z + f(T) L2 + b )              one rounding of the fp32-or-wider sum
The branch reads the unquantized 16-bit X_hat.

Operand layouts follow the kernels' exchange layout: activations [M, K];
weight codes per output column, [N, K] (K contiguous); L1 as [K, r]; L2 [r, N].
"""
from __future__ import annotations

import numpy as np

from .quant import dequantize
from .formats import to_fp16


def down_projection(x_hat: np.ndarray, l1: np.ndarray) -> np.ndarray:
    """T = fp16(X_hat @ L1), float64 accumulation.  x_hat fp16 [M, K], l1 fp16 [K, r]."""
    if l1.shape[1] == 0:
        return np.zeros((x_hat.shape[0], 0), np.float16)
    return to_fp16(x_hat.astype(np.float64) @ l1.astype(np.float64))


def lowbit_gemm(xq_codes, xs, wq_codes, ws, fmt: str) -> np.ndarray:
    """Z = deq(xq) @ deq(wq)^T in float64.  xq_codes [M, K], wq_codes [N, K]."""
    xd = dequantize(xq_codes, xs, fmt)
    wd = dequantize(wq_codes, ws, fmt)
    return xd @ wd.T


def up_projection_output(z: np.ndarray, t: np.ndarray, l2: np.ndarray, bias) -> np.ndarray:
    """Y = fp16(Z + T @ L2 + b), one rounding."""
    acc = np.array(z, dtype=np.float64, copy=True)
    if l2.shape[0]:
        acc += t.astype(np.float64) @ l2.astype(np.float64)
    if bias is not None:
        acc += np.asarray(bias).astype(np.float64)[None, :]
    return to_fp16(acc)


def linear(xq_codes, xs, t, wq_codes, ws, l2, bias, fmt: str) -> np.ndarray:
    """Kernel B's result from Kernel A's outputs (codes, scales, T) and the prepared weight."""
    return up_projection_output(lowbit_gemm(xq_codes, xs, wq_codes, ws, fmt), t, l2, bias)


def w4a16(x: np.ndarray, wq_codes, ws, bias) -> np.ndarray:
    """Weight-only control: Y = fp16( fp16 X @ deq(int4 g64 W)^T + b ), no branch."""
    wd = dequantize(wq_codes, ws, "int4")
    acc = x.astype(np.float64) @ wd.T
    if bias is not None:
        acc += np.asarray(bias).astype(np.float64)[None, :]
    return to_fp16(acc)


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    """GELU, tanh form: 0.5 y (1 + tanh( sqrt(2/pi) (y + 0.044715 y^3) )), float64."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (y + 0.044715 * y * y * y)))


def gelu_smooth(y: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """Glue between the MLP's two linears: fp16( gelu_tanh(Y1) / lambda2 )."""
    return to_fp16(gelu_tanh(np.asarray(y).astype(np.float64)) / lam.astype(np.float64)[None, :])
