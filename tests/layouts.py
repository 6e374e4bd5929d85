"""Device storage layouts of the codes and scales, written on the host for the tests.

The oracle stores every format in the exchange layout: row by row, packed nibbles for INT4
(also for INT4 kept in the 6-bit container), one byte per code for INT8, nibbles for FP4 and
MXFP4.  The kernels keep other layouts in device memory (so that a tile's rows of one 64-wide
chunk of K are one contiguous run); these helpers move the oracle's bytes into them, so that
device buffers can be compared bit for bit without any GPU code in between.  They are test
infrastructure: the layouts are the library's, not the method's.

INT4 in the 6-bit container: code q is the E2M3 bit pattern of q/8 (a subnormal, sign << 5 |
|q|); each run of 32 codes along K (one half of a group of 64) fills 24 bytes, code j in bits
[6j, 6j + 6) of the little-endian run.  On the device a (row, group) has 48 bytes ordered
half 0 bytes 0..15, half 1 bytes 0..15, half 0 bytes 16..23, half 1 bytes 16..23, and the
layout is group-major [K/64][rows][48].
"""
import numpy as np

import oracle


def container_e2m3(codes: np.ndarray) -> np.ndarray:
    """INT4 codes [rows, K] -> the 6-bit container in row order [rows, 3K/4] (each half's 24
    bytes contiguous)."""
    q = np.asarray(codes).astype(np.int64)
    rows, K = q.shape
    f = np.where(q < 0, 32, 0) | np.abs(q)                        # 6-bit fields
    bits = ((f[..., None] >> np.arange(6)) & 1).astype(np.uint8)   # [rows, K, 6], LSB first
    bits = bits.reshape(rows, K // 32, 32 * 6)
    return np.packbits(bits, axis=-1, bitorder="little").reshape(rows, K // 32 * 24)


def uncontainer_e2m3(stored: np.ndarray, K: int) -> np.ndarray:
    """Inverse of container_e2m3."""
    b = np.asarray(stored, np.uint8)
    rows = b.shape[0]
    bits = np.unpackbits(b.reshape(rows, K // 32, 24), axis=-1, bitorder="little").reshape(rows, K, 6)
    f = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)
    mag = f & 31
    return np.where(f & 32, -mag, mag).astype(np.int8)


def dev_codes(stored, fmt):
    """The oracle's stored codes (exchange layout) in the device layout of the format: the
    E2M3 container group-major [K/64][rows][48] in the device's byte order; packed INT4, INT8,
    FP4 and MXFP4 chunk-major [K/64][rows][bytes per chunk]."""
    if fmt in ("int4", "int8", "fp4", "mxfp4"):
        rows = stored.shape[0]
        return np.ascontiguousarray(stored.reshape(rows, -1, 64 if fmt == "int8" else 32).transpose(1, 0, 2))
    assert fmt == "int4_e2m3", fmt
    q = oracle.quant.unpack_int4(stored)
    g = container_e2m3(q)
    rows = g.shape[0]
    g = g.reshape(rows, -1, 48)
    g = np.concatenate([g[..., 0:16], g[..., 24:40], g[..., 16:24], g[..., 40:48]], axis=-1)
    return np.ascontiguousarray(g.transpose(1, 0, 2))


def dev_scales(s, fmt):
    """Scales in the device layout of the format: group-major [K/64][rows] for the INT formats,
    chunk-major [K/64][rows][4] (FP4) or [K/64][rows][2] (MXFP4)."""
    if fmt in ("fp4", "mxfp4"):
        return np.ascontiguousarray(s.reshape(s.shape[0], -1, 4 if fmt == "fp4" else 2).transpose(1, 0, 2))
    assert fmt in ("int4", "int4_e2m3", "int8"), fmt
    return np.ascontiguousarray(s.T)
