"""ctypes binding over libsvdq.so (the C ABI in include/svdq.h).

Argument marshalling only: every computation runs in the HIP kernels of the
library.  Tensors are torch tensors on the current HIP device (PyTorch is used
for device memory and streams); their data pointers and the current stream
are handed to the C entry points of the same names.  The module refuses to
run when the library is missing.
"""
from __future__ import annotations

import ctypes
import functools
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
    "svdq_relayout": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "svdq_linear_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
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


def _raw_stream_fn():
    """A cheap reader of the current stream's handle for a device index: torch's raw-stream
    accessor when it has one (no Stream object per call), else current_stream()."""
    import torch
    fn = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if fn is not None:
        return fn
    return lambda dev: torch.cuda.current_stream(dev).cuda_stream


def _check(name: str, st: int):
    if st != 0:
        raise SvdqError(name, st)


def _need(t, dtype, shape, what):
    """A device tensor of this dtype and shape (None: any), contiguous; else ValueError.  The
    C ABI sees only pointers, so a wrong size would become an out-of-bounds device access:
    every tensor argument is checked here, before any launch."""
    if t is None:
        raise ValueError(f"{what} is required")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if dtype is not None and t.dtype != dtype and not (isinstance(dtype, tuple) and t.dtype in dtype):
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    if shape is not None and t.shape != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _bytes_dtypes():
    """Code tensors are bytes: uint8, or int8 (e.g. INT8 codes as they were computed)."""
    import torch
    return (torch.uint8, torch.int8)


def _absent(t, what, why):
    if t is not None:
        raise ValueError(f"{what} must be None {why}")


def _check_kernel_b(xq, xs, t, wq, ws, l2, bias, K, fmt, y, lam_next=None):
    """Shapes of Kernel B's operands: (M, N, r).  r comes from l2 and must match t."""
    import torch
    if xq is None or wq is None:
        raise ValueError("xq and wq are required")
    M, N = code_rows(xq), code_rows(wq)
    r = 0 if l2 is None else int(l2.shape[0])
    f16 = torch.float16
    _need(xq, _bytes_dtypes(), code_shape(M, K, fmt), "xq")
    _need(xs, scale_dtype(fmt), scale_shape(M, K, fmt), "xs")
    _need(wq, _bytes_dtypes(), code_shape(N, K, fmt), "wq")
    _need(ws, scale_dtype(fmt), scale_shape(N, K, fmt), "ws")
    if r:
        _need(l2, f16, (r, N), "l2")
        _need(t, f16, (M, r), "t")
    else:
        _absent(t, "t", "when l2 is None (no branch)")
    if bias is not None:
        _need(bias, f16, (N,), "bias")
    if y is not None:
        _need(y, f16, (M, N), "y")
    if lam_next is not None:
        _need(lam_next, torch.float32, (N,), "lam_next")
    return M, N, r


def _check_weight(wq, ws, K, fmt):
    import torch
    if wq is None:
        raise ValueError("wq is required")
    N = code_rows(wq)
    _need(wq, _bytes_dtypes(), code_shape(N, K, fmt), "wq")
    _need(ws, scale_dtype(fmt), scale_shape(N, K, fmt), "ws")
    return N


def _check_branch(l1t, l2, K, N):
    """r from l1t [r, K] and l2 [r, N]: both present or both None."""
    import torch
    if (l1t is None) != (l2 is None):
        raise ValueError("l1t and l2 must both be given or both be None")
    if l1t is None:
        return 0
    r = int(l1t.shape[0])
    _need(l1t, torch.float16, (r, K), "l1t")
    _need(l2, torch.float16, (r, N), "l2")
    return r


# ------------------------------------------------------------------ sizes
@functools.lru_cache(maxsize=1024)
def code_row_bytes(K: int, fmt) -> int:
    return int(lib().svdq_code_row_bytes(K, _fmt(fmt)))


@functools.lru_cache(maxsize=4096)
def code_shape(rows: int, K: int, fmt):
    """Shape of a code tensor: chunk-major [K/64, rows, bytes per 64-K chunk] (32 for packed
    INT4, FP4 and MXFP4, 48 for the E2M3 container, 64 for INT8)."""
    name = fmt if isinstance(fmt, str) else FMT_NAMES[int(fmt)]
    return (K // 64, rows, {"int4": 32, "int4_e2m3": 48, "int8": 64, "fp4": 32, "mxfp4": 32}[name])


def code_rows(q) -> int:
    """Rows (tokens or output columns) of a code tensor in either layout."""
    return int(q.shape[1]) if q.dim() == 3 else int(q.shape[0])


def scale_row_entries(K: int, fmt) -> int:
    name = fmt if isinstance(fmt, str) else FMT_NAMES[int(fmt)]
    return K // GROUP[name]


@functools.lru_cache(maxsize=4096)
def scale_shape(rows: int, K: int, fmt):
    """Shape of the scale tensor: group-major [K/64, rows] for the INT formats; chunk-major
    [K/64, rows, 4] (FP4) or [K/64, rows, 2] (MXFP4)."""
    name = fmt if isinstance(fmt, str) else FMT_NAMES[int(fmt)]
    if name in ("int4", "int4_e2m3", "int8"):
        return (K // 64, rows)
    return (K // 64, rows, {"fp4": 4, "mxfp4": 2}[name])


def scale_dtype(fmt):
    import torch
    return torch.uint8 if _fmt(fmt) in (2, 4) else torch.float16   # E4M3 / E8M0 bytes


@functools.lru_cache(maxsize=4096)
def linear_workspace_bytes(M: int, K: int, r: int, fmt) -> int:
    return int(lib().svdq_linear_workspace_bytes(M, K, r, _fmt(fmt)))


@functools.lru_cache(maxsize=4096)
def linear_unfused_workspace_bytes(M: int, N: int, K: int, r: int, fmt) -> int:
    return int(lib().svdq_linear_unfused_workspace_bytes(M, N, K, r, _fmt(fmt)))


# ------------------------------------------------------------------ entry points (same names as the C ABI)
@functools.lru_cache(maxsize=4096)
def quantize_down_workspace_bytes(M: int, K: int, r: int, fmt) -> int:
    return int(lib().svdq_quantize_down_workspace_bytes(M, K, r, _fmt(fmt)))


def _outputs_kernel_a(M, K, r, fmt, dev, xq, xs, t):
    """Kernel A's outputs: every given one is checked before any missing one is allocated."""
    import torch
    if xq is not None:
        _need(xq, _bytes_dtypes(), code_shape(M, K, fmt), "xq")
    if xs is not None:
        _need(xs, scale_dtype(fmt), scale_shape(M, K, fmt), "xs")
    if r:
        if t is not None:
            _need(t, torch.float16, (M, r), "t")
    else:
        _absent(t, "t", "when l1t is None (no branch)")
    if xq is None:
        xq = torch.empty(code_shape(M, K, fmt), dtype=torch.uint8, device=dev)
    if xs is None:
        xs = torch.empty(scale_shape(M, K, fmt), dtype=scale_dtype(fmt), device=dev)
    if r and t is None:
        t = torch.empty((M, r), dtype=torch.float16, device=dev)
    return xq, xs, t


def _workspace_kernel_a(M, K, r, fmt, dev, workspace, no_workspace):
    import torch
    if no_workspace:
        return None, 0
    if workspace is None:
        nb = quantize_down_workspace_bytes(M, K, r, fmt)
        workspace = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    else:
        _need(workspace, None, None, "workspace")
    return workspace, (0 if workspace is None else workspace.numel() * workspace.element_size())


def svdq_quantize_down(x_hat, l1t, fmt, xq=None, xs=None, t=None, workspace=None, no_workspace=False,
                       stream=None):
    """Kernel A.  x_hat fp16 [M, K]; l1t fp16 [r, K] or None.  Returns (xq, xs, t).
    workspace: uint8 device tensor for the sliced-K partial sums (allocated here when None);
    no_workspace=True passes NULL (K not sliced)."""
    import torch
    _need(x_hat, torch.float16, None, "x_hat")
    M, K = x_hat.shape
    r = 0 if l1t is None else int(l1t.shape[0])
    if l1t is not None:
        _need(l1t, torch.float16, (r, K), "l1t")
    dev = x_hat.device
    xq, xs, t = _outputs_kernel_a(M, K, r, fmt, dev, xq, xs, t)
    workspace, ws_bytes = _workspace_kernel_a(M, K, r, fmt, dev, workspace, no_workspace)
    _check("svdq_quantize_down", lib().svdq_quantize_down(
        _p(x_hat), _p(l1t), M, K, r, _fmt(fmt), _p(xq), _p(xs), _p(t), _p(workspace), ws_bytes,
        _stream(stream)))
    return xq, xs, t


def svdq_gemm_w4a4_up(xq, xs, t, wq, ws, l2, bias, K, fmt, y=None, stream=None):
    """Kernel B.  Returns y fp16 [M, N]."""
    import torch
    M, N, r = _check_kernel_b(xq, xs, t, wq, ws, l2, bias, K, fmt, y)
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=xq.device)
    _check("svdq_gemm_w4a4_up", lib().svdq_gemm_w4a4_up(
        _p(xq), _p(xs), _p(t), _p(wq), _p(ws), _p(l2), _p(bias), M, N, K, r, _fmt(fmt), _p(y), _stream(stream)))
    return y


def _layer_args(x, l1t, wq, ws, l2, bias, fmt, y, workspace, need_fn, what="x_hat"):
    """Checks of a whole-layer call's tensors; returns (M, N, K, r, y, workspace, bytes)."""
    import torch
    _need(x, torch.float16, None, what)
    M, K = x.shape
    N = _check_weight(wq, ws, K, fmt)
    r = _check_branch(l1t, l2, K, N)
    if bias is not None:
        _need(bias, torch.float16, (N,), "bias")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(y, torch.float16, (M, N), "y")
    need = need_fn(M, N, K, r)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    else:
        _need(workspace, None, None, "workspace")
    return M, N, K, r, y, workspace, workspace.numel() * workspace.element_size()


def svdq_linear(x_hat, l1t, wq, ws, l2, bias, fmt, workspace=None, y=None, stream=None):
    """Kernel A then Kernel B.  Returns y fp16 [M, N]."""
    M, N, K, r, y, workspace, wb = _layer_args(x_hat, l1t, wq, ws, l2, bias, fmt, y, workspace,
                                               lambda M, N, K, r: linear_workspace_bytes(M, K, r, fmt))
    _check("svdq_linear", lib().svdq_linear(
        _p(x_hat), _p(l1t), _p(wq), _p(ws), _p(l2), _p(bias), M, N, K, r, _fmt(fmt),
        _p(workspace), wb, _p(y), _stream(stream)))
    return y


def _outputs_weight(N, K, fmt, dev, wq, ws):
    """The weight quantizer's outputs: every given one is checked before any missing one is
    allocated."""
    import torch
    if wq is not None:
        _need(wq, _bytes_dtypes(), code_shape(N, K, fmt), "wq")
    if ws is not None:
        _need(ws, scale_dtype(fmt), scale_shape(N, K, fmt), "ws")
    if wq is None:
        wq = torch.empty(code_shape(N, K, fmt), dtype=torch.uint8, device=dev)
    if ws is None:
        ws = torch.empty(scale_shape(N, K, fmt), dtype=scale_dtype(fmt), device=dev)
    return wq, ws


def svdq_quantize_weight(r_t, fmt, wq=None, ws=None, stream=None):
    """Offline: R^T fp32 [N, K] -> (wq, ws)."""
    import torch
    _need(r_t, torch.float32, None, "r_t")
    N, K = r_t.shape
    wq, ws = _outputs_weight(N, K, fmt, r_t.device, wq, ws)
    _check("svdq_quantize_weight", lib().svdq_quantize_weight(
        _p(r_t), N, K, _fmt(fmt), _p(wq), _p(ws), _stream(stream)))
    return wq, ws


def svdq_pack_weight(codes, scales, fmt, wq=None, ws=None, stream=None):
    """Codes int8 [N, K] and fp16 scales [N, K/64] computed elsewhere (e.g. GPTQ) -> (wq, ws) in
    the layouts Kernel B reads (INT formats)."""
    import torch
    _need(codes, torch.int8, None, "codes")
    N, K = codes.shape
    _need(scales, torch.float16, (N, K // 64), "scales")
    wq, ws = _outputs_weight(N, K, fmt, codes.device, wq, ws)
    _check("svdq_pack_weight", lib().svdq_pack_weight(_p(codes), _p(scales), N, K, _fmt(fmt), _p(wq), _p(ws),
                                                      _stream(stream)))
    return wq, ws


def svdq_linear_unfused(x_hat, l1t, wq, ws, l2, bias, fmt, workspace=None, y=None, stream=None):
    """The branch as separate kernels (measurement only).  Returns y fp16 [M, N]."""
    M, N, K, r, y, workspace, wb = _layer_args(
        x_hat, l1t, wq, ws, l2, bias, fmt, y, workspace,
        lambda M, N, K, r: linear_unfused_workspace_bytes(M, N, K, r, fmt))
    _check("svdq_linear_unfused", lib().svdq_linear_unfused(
        _p(x_hat), _p(l1t), _p(wq), _p(ws), _p(l2), _p(bias), M, N, K, r, _fmt(fmt),
        _p(workspace), wb, _p(y), _stream(stream)))
    return y


def svdq_gemm_w4a16(x, wq, ws, bias, y=None, stream=None):
    """W4A16 control.  x fp16 [M, K]; wq, ws: SVDQ_INT4_G64 codes and scales of the N output
    columns (code_shape / scale_shape)."""
    import torch
    _need(x, torch.float16, None, "x")
    M, K = x.shape
    N = _check_weight(wq, ws, K, "int4")
    if bias is not None:
        _need(bias, torch.float16, (N,), "bias")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(y, torch.float16, (M, N), "y")
    _check("svdq_gemm_w4a16", lib().svdq_gemm_w4a16(
        _p(x), _p(wq), _p(ws), _p(bias), M, N, K, _p(y), _stream(stream)))
    return y


def svdq_gelu_tanh_smooth(y, lam, out=None, stream=None):
    """fp16(gelu_tanh(y) / lam) for y fp16 [M, C], lam fp32 [C]."""
    import torch
    _need(y, torch.float16, None, "y")
    M, C = y.shape
    _need(lam, torch.float32, (C,), "lam")
    if out is None:
        out = torch.empty_like(y)
    else:
        _need(out, torch.float16, (M, C), "out")
    _check("svdq_gelu_tanh_smooth", lib().svdq_gelu_tanh_smooth(
        _p(y), _p(lam), M, C, _p(out), _stream(stream)))
    return out


def svdq_quantize_down_smooth(x, lam, l1t, fmt, xq=None, xs=None, t=None, workspace=None, no_workspace=False,
                              stream=None):
    """Kernel A on unsmoothed x fp16 [M, K] with the layer's factors lam fp32 [K]:
    the codes, scales and T of X_hat = fp16(x / lam).  Returns (xq, xs, t).  Workspace as
    for svdq_quantize_down."""
    import torch
    _need(x, torch.float16, None, "x")
    M, K = x.shape
    r = 0 if l1t is None else int(l1t.shape[0])
    _need(lam, torch.float32, (K,), "lam")
    if l1t is not None:
        _need(l1t, torch.float16, (r, K), "l1t")
    dev = x.device
    xq, xs, t = _outputs_kernel_a(M, K, r, fmt, dev, xq, xs, t)
    workspace, ws_bytes = _workspace_kernel_a(M, K, r, fmt, dev, workspace, no_workspace)
    _check("svdq_quantize_down_smooth", lib().svdq_quantize_down_smooth(
        _p(x), _p(lam), _p(l1t), M, K, r, _fmt(fmt), _p(xq), _p(xs), _p(t), _p(workspace), ws_bytes,
        _stream(stream)))
    return xq, xs, t


def svdq_gemm_w4a4_up_gelu_smooth(xq, xs, t, wq, ws, l2, bias, lam_next, K, fmt, y=None, stream=None):
    """Kernel B with an MLP's glue in its epilogue: fp16(gelu(Y) / lam_next), lam_next fp32 [N]."""
    import torch
    if lam_next is None:
        raise ValueError("lam_next is required")
    M, N, r = _check_kernel_b(xq, xs, t, wq, ws, l2, bias, K, fmt, y, lam_next)
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
    M, N, K, r, y, workspace, wb = _layer_args(x, l1t, wq, ws, l2, bias, fmt, y, workspace,
                                               lambda M, N, K, r: linear_workspace_bytes(M, K, r, fmt), "x")
    if lam_in is not None:
        _need(lam_in, torch.float32, (K,), "lam_in")
    if lam_next is not None:
        _need(lam_next, torch.float32, (N,), "lam_next")
    _check("svdq_linear_folded", lib().svdq_linear_folded(
        _p(x), _p(lam_in), _p(l1t), _p(wq), _p(ws), _p(l2), _p(bias), _p(lam_next), M, N, K, r, _fmt(fmt),
        _p(workspace), wb, _p(y), _stream(stream)))
    return y


def canonical_code_shape(rows: int, K: int, fmt):
    """Exchange layout of codes: [rows, K] for INT8, [rows, K/2] (two 4-bit codes a byte) otherwise."""
    return (rows, K if _fmt(fmt) == FORMATS["int8"] else K // 2)


def canonical_scale_shape(rows: int, K: int, fmt):
    name = fmt if isinstance(fmt, str) else FMT_NAMES[int(fmt)]
    return (rows, K // GROUP[name])


def svdq_relayout(codes, scales, K, fmt, to_canonical, codes_out=None, scales_out=None, stream=None):
    """Codes and scales between the exchange layout (row-major, see canonical_code_shape) and the
    format's device layout.  to_canonical=True: device -> exchange.  Returns (codes, scales)."""
    import torch
    if codes is None:
        raise ValueError("codes is required")
    if to_canonical:
        rows = code_rows(codes)
        src_c, src_s = code_shape(rows, K, fmt), scale_shape(rows, K, fmt)
        dst_c, dst_s = canonical_code_shape(rows, K, fmt), canonical_scale_shape(rows, K, fmt)
    else:
        rows = int(codes.shape[0])
        src_c, src_s = canonical_code_shape(rows, K, fmt), canonical_scale_shape(rows, K, fmt)
        dst_c, dst_s = code_shape(rows, K, fmt), scale_shape(rows, K, fmt)
    _need(codes, _bytes_dtypes(), src_c, "codes")
    _need(scales, scale_dtype(fmt), src_s, "scales")
    if codes_out is not None:
        _need(codes_out, _bytes_dtypes(), dst_c, "codes_out")
    if scales_out is not None:
        _need(scales_out, scale_dtype(fmt), dst_s, "scales_out")
    if codes_out is None:
        codes_out = torch.empty(dst_c, dtype=torch.uint8, device=codes.device)
    if scales_out is None:
        scales_out = torch.empty(dst_s, dtype=scale_dtype(fmt), device=codes.device)
    _check("svdq_relayout", lib().svdq_relayout(_p(codes), _p(scales), rows, K, _fmt(fmt), 1 if to_canonical else 0,
                                                _p(codes_out), _p(scales_out), _stream(stream)))
    return codes_out, scales_out


# svdq_linear_noalloc's static device scratch (SVDQ_STATIC_SCRATCH_BYTES in include/svdq.h)
STATIC_SCRATCH_BYTES = 64 << 20


def svdq_linear_noalloc(x_hat, l1t, wq, ws, l2, bias, fmt, y, stream=None):
    """The fused layer with its intermediates in the library's static per-device scratch: no
    device allocation in the library, and none here either (the output y fp16 [M, N] is the
    caller's).  Calls that overlap on one GPU race on the scratch."""
    import torch
    if y is None:
        raise ValueError("y is required (this entry point allocates nothing)")
    _need(x_hat, torch.float16, None, "x_hat")
    M, K = x_hat.shape
    N = _check_weight(wq, ws, K, fmt)
    r = _check_branch(l1t, l2, K, N)
    if bias is not None:
        _need(bias, torch.float16, (N,), "bias")
    _need(y, torch.float16, (M, N), "y")
    _check("svdq_linear_noalloc", lib().svdq_linear_noalloc(
        _p(x_hat), _p(l1t), _p(wq), _p(ws), _p(l2), _p(bias), M, N, K, r, _fmt(fmt), _p(y), _stream(stream)))
    return y


class SvdqLinear:
    """The fused layer prepared for repeated calls (a serving loop, a benchmark's eager steps).

    The weight-side tensors -- residual codes and scales, L1^T, L2, bias -- are checked once
    here and their pointers kept (with references that keep the tensors alive); each call then
    checks only its activations and output, reuses a workspace kept for the largest M seen, and
    makes one svdq_linear call: the same kernels and results as svdq_linear, with a fraction of
    its per-call host work.
    """

    def __init__(self, wq, ws, l1t, l2, bias, K: int, fmt):
        import torch
        self.K, self.fmt, self._F = int(K), fmt, _fmt(fmt)
        self.N = _check_weight(wq, ws, K, fmt)
        self.r = _check_branch(l1t, l2, K, self.N)
        if bias is not None:
            _need(bias, torch.float16, (self.N,), "bias")
        self._keep = (wq, ws, l1t, l2, bias)
        self._ptrs = (_p(l1t), _p(wq), _p(ws), _p(l2), _p(bias))
        self.device = wq.device
        self._dev_index = wq.device.index if wq.device.index is not None else torch.cuda.current_device()
        self._f16 = torch.float16
        self._ws, self._ws_bytes, self._ws_rows = None, 0, -1
        self._fn = lib().svdq_linear
        self._raw_stream = _raw_stream_fn()

    def _workspace(self, M: int):
        if M > self._ws_rows:
            import torch
            nb = max(linear_workspace_bytes(M, self.K, self.r, self.fmt), 16)
            self._ws = torch.empty(nb, dtype=torch.uint8, device=self.device)
            self._ws_bytes, self._ws_rows = nb, M
        return self._ws

    def __call__(self, x_hat, y=None, stream=None):
        """x_hat fp16 [M, K] (smoothed) -> y fp16 [M, N] (allocated when None)."""
        if not (x_hat.is_cuda and x_hat.dtype == self._f16 and x_hat.dim() == 2 and x_hat.shape[1] == self.K
                and x_hat.is_contiguous()):
            _need(x_hat, self._f16, (x_hat.shape[0] if x_hat.dim() == 2 else -1, self.K), "x_hat")
        M = int(x_hat.shape[0])
        if y is None:
            import torch
            y = torch.empty((M, self.N), dtype=self._f16, device=x_hat.device)
        elif not (y.is_cuda and y.dtype == self._f16 and y.shape == (M, self.N) and y.is_contiguous()):
            _need(y, self._f16, (M, self.N), "y")
        ws = self._workspace(M)
        l1t, wq, ws_, l2, b = self._ptrs
        st = self._fn(x_hat.data_ptr(), l1t, wq, ws_, l2, b, M, self.N, self.K, self.r, self._F, ws.data_ptr(),
                      self._ws_bytes, y.data_ptr(), self._raw_stream(self._dev_index) if stream is None else stream)
        if st != 0:
            raise SvdqError("svdq_linear", st)
        return y
