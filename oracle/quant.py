"""Group quantizers of the layer (oracle).

The practice page "sota-314" (section "Do this") fixes per-group symmetric
quantization on both operands: group size 64 with 16-bit scales for INT4,
group size 16 with FP8 scales for NVFP4, and rank 16 at 8 bits.  Groups run
along the reduction axis K for both operands (the only axis along which a
per-chunk rescale of an integer GEMM is possible): per token row for the
activations, per output column for the weight.

INT (qmax = 7 for INT4, 127 for INT8), one group v[0..G-1]:
    a   = max |v|                       (exact)
    s16 = fp16_rne( fp32(a) / fp32(qmax) )   IEEE fp32 division, then RNE to fp16
    s   = float(s16)
    q_k = 0 if s == 0 else clamp( rint_half_even( fp32(v_k) / s ), -qmax, qmax )
Codes are computed against the stored fp16 scale.  INT4 never produces -8.

FP4 (E2M1 codes, group 16, E4M3 scales):
    s8  = e4m3_rne_sat( fp32(a) / 6.0f ),  s = float(s8)
    q_k = 0 if s == 0 else e2m1_nearest_even( fp32(v_k) / s )

MXFP4 (E2M1 codes, group 32, E8M0 scales; OCP Microscaling Formats v1.0, the
format gfx950's block-scaled matrix cores take natively; practice page "sota-314",
section "Conditions": which format wins is a property of the hardware's native
group support):
    e   = floor(log2 a) - 2  (2 = the exponent of E2M1's largest value, 6 = 1.5 * 2^2),
          clamped to [-127, 127]; e = -127 for a = 0
    b8  = e + 127 (the E8M0 byte), X = 2^e
    q_k = e2m1_nearest_even( fp32(v_k) / X )  (exact: X is a power of two), saturating
          at 6: a group's largest values in (6 X, 8 X) become 6 X

Packing of 4-bit codes: two per byte along K, byte b holds code 2b in its low
nibble and code 2b+1 in its high nibble.  INT4 nibbles are two's complement;
E2M1 nibbles are sign<<3 | magnitude index.  INT8 codes are one int8 per byte.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_encode, e2m1_decode, e4m3_encode_rne_sat, e4m3_decode, e8m0_decode

INT4_QMAX = 7
INT8_QMAX = 127


def _groups(v: np.ndarray, G: int) -> np.ndarray:
    rows, K = v.shape
    if K % G:
        raise ValueError(f"K={K} is not a multiple of the group size {G}")
    return v.reshape(rows, K // G, G)


def quantize_int(v: np.ndarray, qmax: int = INT4_QMAX, G: int = 64):
    """Symmetric absmax group quantization along the last axis.

    v: [rows, K] fp16 or fp32.  Returns (codes int8 [rows, K], scales fp16 [rows, K/G]).
    """
    v32 = np.asarray(v).astype(np.float32)
    g = _groups(v32, G)
    a = np.abs(g).max(axis=-1)                                          # exact
    s16 = (a / np.float32(qmax)).astype(np.float32).astype(np.float16)  # fp32 IEEE div, RNE -> fp16
    s = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = g / s[..., None]                                            # fp32 IEEE division
    q = np.clip(np.rint(t), -qmax, qmax)                                # rint = half to even
    q = np.where(s[..., None] == 0, 0, q)
    return q.reshape(v32.shape).astype(np.int8), s16


def quantize_fp4(v: np.ndarray, G: int = 16):
    """E2M1 codes with E4M3 group scales.  Returns (codes uint8 nibbles [rows, K], scales uint8 [rows, K/G])."""
    v32 = np.asarray(v).astype(np.float32)
    g = _groups(v32, G)
    a = np.abs(g).max(axis=-1)
    s8 = e4m3_encode_rne_sat((a / np.float32(6.0)).astype(np.float32))
    s = e4m3_decode(s8).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = g / s[..., None]                                            # fp32 IEEE division
    t = np.where(s[..., None] == 0, 0.0, t)
    codes = e2m1_encode(t.astype(np.float64))
    return codes.reshape(v32.shape).astype(np.uint8), s8


def quantize_mx(v: np.ndarray, G: int = 32):
    """MXFP4: E2M1 codes with E8M0 group scales.  Returns (codes uint8 nibbles [rows, K],
    scales uint8 [rows, K/G])."""
    v32 = np.asarray(v).astype(np.float32)
    g = _groups(v32, G).astype(np.float64)
    a = np.abs(g).max(axis=-1)
    _, ex = np.frexp(a)                          # a = m 2^ex with m in [0.5, 1): floor(log2 a) = ex - 1
    e = np.where(a > 0, ex - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    t = np.ldexp(g, -e[..., None])               # v / 2^e, exact
    codes = e2m1_encode(t)
    return codes.reshape(v32.shape).astype(np.uint8), (e + 127).astype(np.uint8)


def dequant_mx(codes: np.ndarray, scales8: np.ndarray, G: int = 32) -> np.ndarray:
    q = e2m1_decode(codes)
    s = e8m0_decode(scales8)
    return (q.reshape(q.shape[0], -1, G) * s[..., None]).reshape(q.shape)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[rows, K] 4-bit codes (int8 two's complement or uint8 nibbles) -> uint8 [rows, K/2]."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """uint8 [rows, K/2] -> int8 codes [rows, K] (two's complement nibbles)."""
    p = np.asarray(packed).astype(np.int64)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.int64)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [rows, K/2] -> uint8 nibbles [rows, K] (no sign interpretation)."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2], out[:, 1::2] = p & 0xF, p >> 4
    return out


def dequant_int(codes: np.ndarray, scales16: np.ndarray, G: int = 64) -> np.ndarray:
    """q * s in float64 (exact: a small integer times an fp16)."""
    q = np.asarray(codes).astype(np.float64)
    s = np.asarray(scales16).astype(np.float64)
    return (q.reshape(q.shape[0], -1, G) * s[..., None]).reshape(q.shape)


def dequant_fp4(codes: np.ndarray, scales8: np.ndarray, G: int = 16) -> np.ndarray:
    q = e2m1_decode(codes)
    s = e4m3_decode(scales8)
    return (q.reshape(q.shape[0], -1, G) * s[..., None]).reshape(q.shape)


# ------------------------------------------------------------------ format table
FORMATS = {
    # name: (group size, bits per code, scale dtype)
    "int4": (64, 4, "fp16"),
    "int8": (64, 8, "fp16"),
    "fp4": (16, 4, "e4m3"),
    "int4_e2m3": (64, 4, "fp16"),   # INT4 (the library keeps these codes in a 6-bit container)
    "mxfp4": (32, 4, "e8m0"),
}


def quantize(v: np.ndarray, fmt: str):
    """Quantize rows of v in the named format.

    Returns (codes, scales, stored) where `stored` is the exchange layout, row by
    row: packed nibbles for int4 (also "int4_e2m3", the same codes, which the
    library keeps in a storage container of its own), fp4 and mxfp4, one byte
    per code for int8.
    """
    if fmt == "int4":
        q, s = quantize_int(v, INT4_QMAX, 64)
        return q, s, pack_nibbles(q)
    if fmt == "int8":
        q, s = quantize_int(v, INT8_QMAX, 64)
        return q, s, q.copy()
    if fmt == "int4_e2m3":
        q, s = quantize_int(v, INT4_QMAX, 64)
        return q, s, pack_nibbles(q)
    if fmt == "fp4":
        q, s = quantize_fp4(v, 16)
        return q, s, pack_nibbles(q)
    if fmt == "mxfp4":
        q, s = quantize_mx(v, 32)
        return q, s, pack_nibbles(q)
    raise ValueError(fmt)


def dequantize(codes, scales, fmt: str) -> np.ndarray:
    if fmt in ("int4", "int8", "int4_e2m3"):
        return dequant_int(codes, scales, 64)
    if fmt == "fp4":
        return dequant_fp4(codes, scales, 16)
    if fmt == "mxfp4":
        return dequant_mx(codes, scales, 32)
    raise ValueError(fmt)
