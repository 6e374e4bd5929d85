"""Offline preparation of one SVDQuant layer (host side, not on the timed path).

Practice page "sota-314", section "Do this": smooth the activation outliers
into the weight, take the SVD of the smoothed weight, keep the top r singular
directions as a 16-bit branch and quantize only the residual.  Reading note
"note-257", section "Key results": L1 = U Sigma[:, :r], L2 = V[:r, :].

Host arithmetic (float64 LAPACK SVD; the smoothing factor and the smoothed
activations in fp32 then fp16):
    lambda_j = sqrt(fp32(max_i |X_ij|) / fp32(max_n |W_jn|))   (1 if either is 0)
    X_hat    = fp16(fp32(X) / lambda)
    W_hat    = lambda W                                     (float64)
    L1 = fp16(U_r Sigma_r), L2 = fp16(V_r^T), R = W_hat - L1 L2   (float64 -> fp32)
The residual's codes and scales are then produced on the GPU by
svdq_quantize_weight.  The device tensors are laid out the way the kernels
read them: L1^T [r, K], L2 [r, N], codes / scales per output column [N, ...].
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


def _channel_factor(x_cal: np.ndarray, w: np.ndarray) -> np.ndarray:
    act_max = np.max(np.abs(np.asarray(x_cal, dtype=np.float32)), axis=0)
    wt_max = np.max(np.abs(np.asarray(w, dtype=np.float32)), axis=1)
    lam = np.ones(act_max.shape, dtype=np.float32)
    nz = np.logical_and(act_max > 0, wt_max > 0)
    lam[nz] = np.sqrt(act_max[nz] / wt_max[nz])
    return lam


@dataclass
class HostLayer:
    """Host-side result of the offline preparation."""
    lam: np.ndarray       # fp32 [K]
    l1t: np.ndarray       # fp16 [r, K]
    l2: np.ndarray        # fp16 [r, N]
    r_t: np.ndarray       # fp32 [N, K], residual transposed (K contiguous per output column)
    bias: np.ndarray      # fp16 [N]

    def smooth(self, x: np.ndarray) -> np.ndarray:
        """Smoothed activations fp16(fp32(x) / lambda)."""
        return (np.asarray(x, dtype=np.float32) / self.lam).astype(np.float16)


def prepare_host(x_cal: np.ndarray, w: np.ndarray, bias: np.ndarray, r: int) -> HostLayer:
    """Smoothing from calibration activations x_cal [M, K], SVD split of lambda W [K, N]."""
    lam = _channel_factor(x_cal, w)
    w_s = np.asarray(w, dtype=np.float64) * lam.astype(np.float64)[:, None]
    K, N = w_s.shape
    u, sig, vt = np.linalg.svd(w_s, full_matrices=False)
    if r:
        l1 = (u[:, :r] * sig[None, :r]).astype(np.float16)
        l2 = vt[:r].astype(np.float16)
        resid = w_s - np.matmul(l1.astype(np.float64), l2.astype(np.float64))
    else:
        l1 = np.zeros((K, 0), np.float16)
        l2 = np.zeros((0, N), np.float16)
        resid = w_s
    return HostLayer(lam, np.ascontiguousarray(l1.T), l2, np.ascontiguousarray(resid.astype(np.float32).T),
                     np.asarray(bias, dtype=np.float16))


def attach_lora(h: HostLayer, a: np.ndarray, b: np.ndarray, scale: float = 1.0) -> HostLayer:
    """The layer with a LoRA adapter (delta W = scale A B; A [K, ra], B [ra, N]) in its 16-bit
    branch ("sota-314", "Known implementations": the authors' engine attaches adapters and keeps
    the quantized weights as they are).
    X A B = X_hat diag(lambda) A B, so the branch grows to
        L1^T' = [L1^T; fp16(diag(lambda) A)^T],   L2' = [L2; fp16(scale B)]
    (products in float64, one rounding each), zero rows padding the rank to a multiple of 16
    (the kernels' granularity; a zero row adds exactly 0).  The residual R is unchanged, so
    its device codes can be reused (with_branch)."""
    K, ra = a.shape
    N = h.l2.shape[1]
    la_t = (h.lam.astype(np.float64)[:, None] * np.asarray(a, np.float64)).astype(np.float16).T
    lb = (float(scale) * np.asarray(b, np.float64)).astype(np.float16)
    r = h.l1t.shape[0] + ra
    pad = (-r) % 16
    l1t = np.concatenate([h.l1t, la_t, np.zeros((pad, K), np.float16)], axis=0)
    l2 = np.concatenate([h.l2, lb, np.zeros((pad, N), np.float16)], axis=0)
    if l1t.shape[0] > 64:
        raise ValueError(f"branch rank {l1t.shape[0]} exceeds the kernels' 64")
    return HostLayer(h.lam, np.ascontiguousarray(l1t), np.ascontiguousarray(l2), h.r_t, h.bias)


def gptq_residual(h: HostLayer, x_cal_hat: np.ndarray, fmt: str, damp: float = 0.01):
    """GPTQ codes of the residual ("sota-314", "Do this": the residual weights are quantized
    with GPTQ in the authors' pipeline, not to nearest; Frantar et al. 2022, "GPTQ", Algorithm 1, without
    its lazy batching, which only regroups the same updates).  x_cal_hat: smoothed calibration
    activations [M, K] (the inputs R multiplies).  Each input channel in turn is rounded with
    the round-to-nearest rule (fp16 group scale from the group's current weights at its first
    channel) and its error moved onto the channels not yet rounded through the upper
    Cholesky factor of the damped inverse Hessian of 2 X^T X (float64).  INT formats only.
    Returns (codes int8 [N, K], scales fp16 [N, K/64]) for svdq_pack_weight."""
    if fmt not in ("int4", "int4_e2m3", "int8"):
        raise ValueError(f"GPTQ codes are produced for the INT formats, not {fmt}")
    qmax = np.float32(127.0 if fmt == "int8" else 7.0)
    w = np.asarray(h.r_t, dtype=np.float64).copy()       # [N, K]
    x = np.asarray(x_cal_hat, dtype=np.float64)
    hess = 2.0 * x.T @ x
    K = hess.shape[0]
    idle = np.diag(hess) == 0                             # channels never active: weight 0
    hess[idle, idle] = 1.0
    w[:, idle] = 0.0
    hess[np.diag_indices(K)] += damp * np.mean(np.diag(hess))
    chol_u = np.linalg.cholesky(np.linalg.inv(hess)).T   # H^-1 = U^T U, U upper
    codes = np.zeros(w.shape, np.int8)
    scales = np.zeros((w.shape[0], K // 64), np.float16)
    for j in range(K):
        grp = j // 64
        if j % 64 == 0:
            amax = np.abs(w[:, j:j + 64].astype(np.float32)).max(axis=1)
            scales[:, grp] = (amax / qmax).astype(np.float32).astype(np.float16)
        s32 = scales[:, grp].astype(np.float32)
        col = w[:, j].astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            quot = np.where(s32 == 0, np.float32(0.0), col / s32)
        q = np.clip(np.rint(quot), -qmax, qmax).astype(np.int8)
        codes[:, j] = q
        err = (w[:, j] - q.astype(np.float64) * s32.astype(np.float64)) / chol_u[j, j]
        w[:, j + 1:] -= np.outer(err, chol_u[j, j + 1:])
    return codes, scales


@dataclass
class DeviceLayer:
    """The prepared layer resident in device memory, ready for svdq_linear."""
    fmt: str
    K: int
    N: int
    r: int
    l1t: Optional[object]   # torch fp16 [r, K] or None
    l2: Optional[object]    # torch fp16 [r, N] or None
    wq: object              # torch uint8 codes [N, ...]
    ws: object              # torch scales [N, ...]
    bias: Optional[object]  # torch fp16 [N]
    lam: object             # torch fp32 [K]


def to_device(h: HostLayer, fmt: str, device="cuda", stream=None) -> DeviceLayer:
    """Upload the host layer and quantize its residual on the GPU."""
    import torch
    from .binding import svdq_quantize_weight
    r = h.l1t.shape[0]
    N, K = h.r_t.shape
    r_t = torch.from_numpy(h.r_t).to(device)
    wq, ws = svdq_quantize_weight(r_t, fmt, stream=stream)
    l1t = torch.from_numpy(h.l1t).to(device) if r else None
    l2 = torch.from_numpy(h.l2).to(device) if r else None
    bias = torch.from_numpy(h.bias).to(device)
    lam = torch.from_numpy(h.lam).to(device)
    del r_t
    return DeviceLayer(fmt, K, N, r, l1t, l2, wq, ws, bias, lam)


def to_device_packed(h: HostLayer, fmt: str, codes: np.ndarray, scales: np.ndarray, device="cuda",
                     stream=None) -> DeviceLayer:
    """Upload the host layer with residual codes computed on the host (e.g. gptq_residual),
    packed into Kernel B's layout by svdq_pack_weight."""
    import torch
    from .binding import svdq_pack_weight
    r = h.l1t.shape[0]
    N, K = h.r_t.shape
    wq, ws = svdq_pack_weight(torch.from_numpy(np.ascontiguousarray(codes)).to(device),
                              torch.from_numpy(np.ascontiguousarray(scales)).to(device), fmt, stream=stream)
    l1t = torch.from_numpy(h.l1t).to(device) if r else None
    l2 = torch.from_numpy(h.l2).to(device) if r else None
    return DeviceLayer(fmt, K, N, r, l1t, l2, wq, ws, torch.from_numpy(h.bias).to(device),
                       torch.from_numpy(h.lam).to(device))


def with_branch(d: DeviceLayer, h: HostLayer, device="cuda") -> DeviceLayer:
    """The device layer with the branch of host layer h (e.g. after attach_lora): new L1^T and
    L2 uploads, the residual's codes and scales reused as they are (no re-quantization)."""
    import torch
    r = h.l1t.shape[0]
    l1t = torch.from_numpy(h.l1t).to(device) if r else None
    l2 = torch.from_numpy(h.l2).to(device) if r else None
    return DeviceLayer(d.fmt, d.K, d.N, r, l1t, l2, d.wq, d.ws, d.bias, d.lam)
