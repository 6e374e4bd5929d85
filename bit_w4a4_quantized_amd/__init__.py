"""SVDQuant W4A4 linear layer for AMD Instinct MI355X (gfx950).

The layer runs in hand-written HIP kernels behind a C ABI (include/svdq.h,
built into libsvdq.so in this directory); `binding` is the ctypes layer over
it and `prepare` the offline layer preparation.
"""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    svdq_quantize_down, svdq_gemm_w4a4_up, svdq_linear, svdq_quantize_weight,
    svdq_linear_unfused, svdq_gemm_w4a16, svdq_gelu_tanh_smooth, SvdqError,
)
