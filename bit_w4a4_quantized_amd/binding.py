"""ctypes binding over libsvdq.so (the C ABI in include/svdq.h).

Argument marshalling only: every computation runs in the HIP kernels of the
library.  Tensors are torch tensors on the current HIP device (PyTorch is used
for device memory and streams); their data pointers and the current stream
are handed to the C entry points of the same names.  The module refuses to
run when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# SVDQ_LIBRARY may name another build of the same library (same ABI), e.g. a tuning variant.
LIB_PATH = os.environ.get("SVDQ_LIBRARY") or os.path.join(HERE, "libsvdq.so")

FORMATS = {"int4": 0, "int8": 1, "fp4": 2, "int4_e2m3": 3, "mxfp4": 4}
GROUP = {"int4": 64, "int8": 64, "fp4": 16, "int4_e2m3": 64, "mxfp4": 32}
FMT_NAMES = {v: k for k, v in FORMATS.items()}

_lib = None

_c_int, _c_size, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

_SIGS = {
    "svdq_code_row_bytes": (_c_size, [_c_int, _c_int]),
    "svdq_scale_row_bytes": (_c_size, [_c_int, _c_int]),
    "svdq_quantize_down": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "svdq_quantize_down_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "svdq_gemm_w4a4_up": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "svdq_linear_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "svdq_linear": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _c_size, _vp, _vp]),
    "svdq_quantize_weight": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "svdq_pack_weight": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "svdq_linear_unfused_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int]),
    "svdq_linear_unfused": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _c_size, _vp, _vp]),
    "svdq_gemm_w4a16": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "svdq_gelu_tanh_smooth": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp]),
    "svdq_quantize_down_smooth": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                           _c_size, _vp]),
    "svdq_gemm_w4a4_up_gelu_smooth": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int,
                                               _c_int, _c_int, _vp, _vp]),
    "svdq_linear_folded": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _vp, _c_size, _vp, _vp]),
    "svdq_status_string": (ctypes.c_char_p, [_c_int]),
    "svdq_version": (ctypes.c_char_p, []),
}


class SvdqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libsvdq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_w4a4_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().svdq_status_string(s).decode()


def version() -> str:
    return lib().svdq_version().decode()


def _fmt(fmt) -> int:
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(name: str, st: int):
    if st != 0:
        raise SvdqError(name, st)


def _need(t, dtype, shape, what):
    import torch
    if t is None:
        raise ValueError(f"{what} is required")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


# ------------------------------------------------------------------ sizes
def code_row_bytes(K: int, fmt) -> int:
    return int(lib().svdq_code_row_bytes(K, _fmt(fmt)))


def code_shape(rows: int, K: int, fmt):
    """Shape of a code tensor: row-major [rows, K/2] for packed INT4; chunk-major
    [K/64, rows, bytes per 64-K chunk] otherwise (48 for the E2M3 container, 64 for INT8, 32
    for FP4 and MXFP4)."""
    name = fmt if isinstance(fmt, str) else FMT_NAMES[int(fmt)]
    if name == "int4":
        return (rows, code_row_bytes(K, fmt))
    return (K // 64, rows, {"int4_e2m3": 48, "int8": 64, "fp4": 32, "mxfp4": 32}[name])


def code_rows(q) -> int:
    """Rows (tokens or output columns) of a code tensor in either layout."""
    return int(q.shape[1]) if q.dim() == 3 else int(q.shape[0])


def scale_row_entries(K: int, fmt) -> int:
    name = fmt if isinstance(fmt, str) else FMT_NAMES[int(fmt)]
    return K // GROUP[name]


def scale_shape(rows: int, K: int, fmt):
    """Shape of the scale tensor: row-major [rows, K/64] for packed INT4; group-major
    [K/64, rows] for the E2M3 container and INT8; chunk-major [K/64, rows, 4] (FP4) or
    [K/64, rows, 2] (MXFP4)."""
    name = fmt if isinstance(fmt, str) else FMT_NAMES[int(fmt)]
    if name == "int4":
        return (rows, K // 64)
    if name in ("int4_e2m3", "int8"):
        return (K // 64, rows)
    return (K // 64, rows, {"fp4": 4, "mxfp4": 2}[name])


def scale_dtype(fmt):
    import torch
    return torch.uint8 if _fmt(fmt) in (2, 4) else torch.float16   # E4M3 / E8M0 bytes


def linear_workspace_bytes(M: int, K: int, r: int, fmt) -> int:
    return int(lib().svdq_linear_workspace_bytes(M, K, r, _fmt(fmt)))


def linear_unfused_workspace_bytes(M: int, N: int, K: int, r: int, fmt) -> int:
    return int(lib().svdq_linear_unfused_workspace_bytes(M, N, K, r, _fmt(fmt)))


# ------------------------------------------------------------------ entry points (same names as the C ABI)
def quantize_down_workspace_bytes(M: int, K: int, r: int, fmt) -> int:
    return int(lib().svdq_quantize_down_workspace_bytes(M, K, r, _fmt(fmt)))


def svdq_quantize_down(x_hat, l1t, fmt, xq=None, xs=None, t=None, workspace=None, no_workspace=False,
                       stream=None):
    """Kernel A.  x_hat fp16 [M, K]; l1t fp16 [r, K] or None.  Returns (xq, xs, t).
    workspace: uint8 device tensor for the sliced-K partial sums (allocated here when None);
    no_workspace=True passes NULL (K not sliced)."""
    import torch
    M, K = x_hat.shape
    r = 0 if l1t is None else l1t.shape[0]
    _need(x_hat, torch.float16, None, "x_hat")
    if l1t is not None:
        _need(l1t, torch.float16, (r, K), "l1t")
    dev = x_hat.device
    if xq is None:
        xq = torch.empty(code_shape(M, K, fmt), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty(scale_shape(M, K, fmt), dtype=scale_dtype(fmt), device=dev)
    if r and t is None:
        t = torch.empty((M, r), dtype=torch.float16, device=dev)
    if no_workspace:
        workspace = None
    elif workspace is None:
        nb = quantize_down_workspace_bytes(M, K, r, fmt)
        workspace = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("svdq_quantize_down", lib().svdq_quantize_down(
        _p(x_hat), _p(l1t), M, K, r, _fmt(fmt), _p(xq), _p(xs), _p(t), _p(workspace), ws_bytes,
        _stream(stream)))
    return xq, xs, t


def svdq_gemm_w4a4_up(xq, xs, t, wq, ws, l2, bias, K, fmt, y=None, stream=None):
    """Kernel B.  Returns y fp16 [M, N]."""
    import torch
    M = code_rows(xq)
    N = code_rows(wq)
    r = 0 if l2 is None else l2.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=xq.device)
    _check("svdq_gemm_w4a4_up", lib().svdq_gemm_w4a4_up(
        _p(xq), _p(xs), _p(t), _p(wq), _p(ws), _p(l2), _p(bias), M, N, K, r, _fmt(fmt), _p(y), _stream(stream)))
    return y


def svdq_linear(x_hat, l1t, wq, ws, l2, bias, fmt, workspace=None, y=None, stream=None):
    """Kernel A then Kernel B.  Returns y fp16 [M, N]."""
    import torch
    M, K = x_hat.shape
    N = code_rows(wq)
    r = 0 if l1t is None else l1t.shape[0]
    need = linear_workspace_bytes(M, K, r, fmt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x_hat.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x_hat.device)
    _check("svdq_linear", lib().svdq_linear(
        _p(x_hat), _p(l1t), _p(wq), _p(ws), _p(l2), _p(bias), M, N, K, r, _fmt(fmt),
        _p(workspace), workspace.numel() * workspace.element_size(), _p(y), _stream(stream)))
    return y


def svdq_quantize_weight(r_t, fmt, wq=None, ws=None, stream=None):
    """Offline: R^T fp32 [N, K] -> (wq, ws)."""
    import torch
    N, K = r_t.shape
    _need(r_t, torch.float32, None, "r_t")
    if wq is None:
        wq = torch.empty(code_shape(N, K, fmt), dtype=torch.uint8, device=r_t.device)
    if ws is None:
        ws = torch.empty(scale_shape(N, K, fmt), dtype=scale_dtype(fmt), device=r_t.device)
    _check("svdq_quantize_weight", lib().svdq_quantize_weight(
        _p(r_t), N, K, _fmt(fmt), _p(wq), _p(ws), _stream(stream)))
    return wq, ws


def svdq_pack_weight(codes, scales, fmt, wq=None, ws=None, stream=None):
    """Codes int8 [N, K] and fp16 scales [N, K/64] computed elsewhere (e.g. GPTQ) -> (wq, ws) in
    the layouts Kernel B reads (INT formats)."""
    import torch
    N, K = codes.shape
    _need(codes, torch.int8, None, "codes")
    _need(scales, torch.float16, (N, K // 64), "scales")
    if wq is None:
        wq = torch.empty(code_shape(N, K, fmt), dtype=torch.uint8, device=codes.device)
    if ws is None:
        ws = torch.empty(scale_shape(N, K, fmt), dtype=scale_dtype(fmt), device=codes.device)
    _check("svdq_pack_weight", lib().svdq_pack_weight(_p(codes), _p(scales), N, K, _fmt(fmt), _p(wq), _p(ws),
                                                      _stream(stream)))
    return wq, ws


def svdq_linear_unfused(x_hat, l1t, wq, ws, l2, bias, fmt, workspace=None, y=None, stream=None):
    """The branch as separate kernels (measurement only).  Returns y fp16 [M, N]."""
    import torch
    M, K = x_hat.shape
    N = code_rows(wq)
    r = 0 if l1t is None else l1t.shape[0]
    need = linear_unfused_workspace_bytes(M, N, K, r, fmt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x_hat.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x_hat.device)
    _check("svdq_linear_unfused", lib().svdq_linear_unfused(
        _p(x_hat), _p(l1t), _p(wq), _p(ws), _p(l2), _p(bias), M, N, K, r, _fmt(fmt),
        _p(workspace), workspace.numel() * workspace.element_size(), _p(y), _stream(stream)))
    return y


def svdq_gemm_w4a16(x, wq, ws, bias, y=None, stream=None):
    """W4A16 control.  x fp16 [M, K]; wq uint8 [N, K/2]; ws fp16 [N, K/64]."""
    import torch
    M, K = x.shape
    N = code_rows(wq)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check("svdq_gemm_w4a16", lib().svdq_gemm_w4a16(
        _p(x), _p(wq), _p(ws), _p(bias), M, N, K, _p(y), _stream(stream)))
    return y


def svdq_gelu_tanh_smooth(y, lam, out=None, stream=None):
    """fp16(gelu_tanh(y) / lam) for y fp16 [M, C], lam fp32 [C]."""
    import torch
    M, C = y.shape
    if out is None:
        out = torch.empty_like(y)
    _check("svdq_gelu_tanh_smooth", lib().svdq_gelu_tanh_smooth(
        _p(y), _p(lam), M, C, _p(out), _stream(stream)))
    return out


def svdq_quantize_down_smooth(x, lam, l1t, fmt, xq=None, xs=None, t=None, workspace=None, no_workspace=False,
                              stream=None):
    """Kernel A on unsmoothed x fp16 [M, K] with the layer's factors lam fp32 [K]:
    the codes, scales and T of X_hat = fp16(x / lam).  Returns (xq, xs, t).  Workspace as
    for svdq_quantize_down."""
    import torch
    M, K = x.shape
    r = 0 if l1t is None else l1t.shape[0]
    _need(x, torch.float16, None, "x")
    _need(lam, torch.float32, (K,), "lam")
    if l1t is not None:
        _need(l1t, torch.float16, (r, K), "l1t")
    dev = x.device
    if xq is None:
        xq = torch.empty(code_shape(M, K, fmt), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty(scale_shape(M, K, fmt), dtype=scale_dtype(fmt), device=dev)
    if r and t is None:
        t = torch.empty((M, r), dtype=torch.float16, device=dev)
    if no_workspace:
        workspace = None
    elif workspace is None:
        nb = quantize_down_workspace_bytes(M, K, r, fmt)
        workspace = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("svdq_quantize_down_smooth", lib().svdq_quantize_down_smooth(
        _p(x), _p(lam), _p(l1t), M, K, r, _fmt(fmt), _p(xq), _p(xs), _p(t), _p(workspace), ws_bytes,
        _stream(stream)))
    return xq, xs, t


def svdq_gemm_w4a4_up_gelu_smooth(xq, xs, t, wq, ws, l2, bias, lam_next, K, fmt, y=None, stream=None):
    """Kernel B with an MLP's glue in its epilogue: fp16(gelu(Y) / lam_next), lam_next fp32 [N]."""
    import torch
    M = code_rows(xq)
    N = code_rows(wq)
    r = 0 if l2 is None else l2.shape[0]
    _need(lam_next, torch.float32, (N,), "lam_next")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=xq.device)
    _check("svdq_gemm_w4a4_up_gelu_smooth", lib().svdq_gemm_w4a4_up_gelu_smooth(
        _p(xq), _p(xs), _p(t), _p(wq), _p(ws), _p(l2), _p(bias), _p(lam_next), M, N, K, r, _fmt(fmt), _p(y),
        _stream(stream)))
    return y


def svdq_linear_folded(x, lam_in, l1t, wq, ws, l2, bias, lam_next, fmt, workspace=None, y=None, stream=None):
    """The layer with either fold: lam_in fp32 [K] (x unsmoothed) and/or lam_next fp32 [N]
    (output fp16(gelu(Y) / lam_next)); None for a fold not taken.  Returns y fp16 [M, N]."""
    import torch
    M, K = x.shape
    N = code_rows(wq)
    r = 0 if l1t is None else l1t.shape[0]
    if lam_in is not None:
        _need(lam_in, torch.float32, (K,), "lam_in")
    if lam_next is not None:
        _need(lam_next, torch.float32, (N,), "lam_next")
    need = linear_workspace_bytes(M, K, r, fmt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _check("svdq_linear_folded", lib().svdq_linear_folded(
        _p(x), _p(lam_in), _p(l1t), _p(wq), _p(ws), _p(l2), _p(bias), _p(lam_next), M, N, K, r, _fmt(fmt),
        _p(workspace), workspace.numel() * workspace.element_size(), _p(y), _stream(stream)))
    return y
