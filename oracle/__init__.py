"""CPU oracle for the SVDQuant W4A4 linear layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the layer
computes, written from the method's description (SVDQuant: Li, Lin, Zhang,
Cai, Li, Guo, Xie, Meng, Zhu, Han 2024, as recorded in the "sota-314"
practice page, section "Do this", and the "note-257" reading note, section
"Key results").  Only the tests, the smoke check and the benchmark's CPU
baseline may import it; the GPU library never does, and the two share no
code.

Modules:
  formats  -- fp16 / E4M3 / E2M1 number formats (definitions)
  quant    -- group quantizers (INT4/INT8 absmax, FP4 E2M1 with E4M3 scales), packing
  prep     -- offline setup: smoothing, truncated SVD, residual
  forward  -- the layer: down projection, low-bit GEMM, up projection, bias;
              the W4A16 control; the GELU(tanh) + smoothing glue
  brute    -- independent float64 loops of the per-group integer form (tiny shapes)
  gptq     -- GPTQ rounding of the residual (error compensation over the Hessian of X_hat)

Every function is pinned by a CPU test against something other than itself
(closed forms, worked special cases, library routines, exhaustive tables or
brute force); none is "parity unpinned".
"""
from . import formats, quant, prep, forward, brute, gptq  # noqa: F401
