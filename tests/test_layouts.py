"""The tests' host-side device layouts (tests/layouts.py), checked on the CPU against the
definitions they restate: the E2M3 bit pattern of q/8 for the 6-bit container, and round
trips of every layout."""
import numpy as np

import oracle
from tests.layouts import container_e2m3, dev_codes, dev_scales, uncontainer_e2m3


def _e2m3_value(f):
    """E2M3 from its definition: sign bit 5, exponent bits 4..3 (bias 1), mantissa bits 2..0."""
    s = -1.0 if f & 32 else 1.0
    e, m = (f >> 3) & 3, f & 7
    return s * (m / 8.0 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 1))


def test_e2m3_container_round_trip_and_values(rng):
    q = rng.integers(-7, 8, (6, 256)).astype(np.int8)
    st = container_e2m3(q)
    assert st.shape == (6, 256 * 3 // 4)
    assert np.array_equal(uncontainer_e2m3(st, 256), q)
    # each 6-bit field decodes (as E2M3) to q/8; field j of a 32-code run sits at bits 6j..6j+5
    bits = np.unpackbits(st[0, :24], bitorder="little")
    for j in range(32):
        f = int(sum(int(bits[6 * j + i]) << i for i in range(6)))
        assert _e2m3_value(f) == q[0, j] / 8.0
    # the second run (codes 32..63 of group 0) starts at byte 24
    bits = np.unpackbits(st[0, 24:48], bitorder="little")
    f = int(sum(int(bits[i]) << i for i in range(6)))
    assert _e2m3_value(f) == q[0, 32] / 8.0


def test_device_container_order(rng):
    """Group-major [K/64][rows][48]; per (row, group): half 0 bytes 0..15, half 1 bytes 0..15,
    then both halves' bytes 16..23."""
    rows, K = 5, 192
    q = rng.integers(-7, 8, (rows, K)).astype(np.int8)
    d = dev_codes(oracle.quant.pack_nibbles(q), "int4_e2m3")
    assert d.shape == (K // 64, rows, 48)
    c = container_e2m3(q).reshape(rows, K // 64, 2, 24)     # [row, group, half, byte]
    for g in range(K // 64):
        for m in range(rows):
            assert np.array_equal(d[g, m, 0:16], c[m, g, 0, 0:16])
            assert np.array_equal(d[g, m, 16:32], c[m, g, 1, 0:16])
            assert np.array_equal(d[g, m, 32:40], c[m, g, 0, 16:24])
            assert np.array_equal(d[g, m, 40:48], c[m, g, 1, 16:24])


def test_chunk_major_layouts(rng):
    rows, K = 3, 256
    b8 = rng.integers(-127, 128, (rows, K)).astype(np.int8)
    d = dev_codes(b8, "int8")
    assert d.shape == (K // 64, rows, 64) and np.array_equal(d[2, 1], b8[1, 128:192])
    nib = oracle.quant.pack_nibbles(rng.integers(0, 16, (rows, K)).astype(np.uint8))
    for fmt in ("int4", "fp4", "mxfp4"):
        d = dev_codes(nib, fmt)
        assert d.shape == (K // 64, rows, 32) and np.array_equal(d[3, 2], nib[2, 96:128])
    s16 = rng.standard_normal((rows, K // 64)).astype(np.float16)
    for fmt in ("int4", "int4_e2m3", "int8"):
        assert np.array_equal(dev_scales(s16, fmt), s16.T)
    e4 = rng.integers(0, 256, (rows, K // 16)).astype(np.uint8)
    assert np.array_equal(dev_scales(e4, "fp4")[1, 2], e4[2, 4:8])
    e8 = rng.integers(0, 256, (rows, K // 32)).astype(np.uint8)
    assert np.array_equal(dev_scales(e8, "mxfp4")[3, 0], e8[0, 6:8])
