"""The package's offline preparation against the oracle's offline setup (CPU).

The two are written separately; on the same raw layer they must agree bit for
bit (same fp32/fp16 rounding points, same LAPACK routine), so the GPU path and
the oracle see the same prepared layer whichever of the two made it.
"""
import numpy as np
import pytest

from bit_w4a4_quantized_amd.prepare import prepare_host
from oracle import prep
from synth import draw_layer, LayerShape


@pytest.mark.parametrize("shape", [LayerShape("a", 128, 256, 256, 32, "int4", 1000, 8),
                                   LayerShape("b", 64, 192, 96, 16, "int8", 5, 4),
                                   LayerShape("c", 33, 128, 48, 0, "int4", 6, 4)])
def test_product_prep_equals_oracle_prep(shape):
    raw = draw_layer(shape)
    h = prepare_host(raw.x, raw.w, raw.b, shape.r)
    o = prep.prepare_layer(raw.x, raw.w, raw.b, shape.r)
    assert np.array_equal(h.lam.view(np.uint32), o.lam.view(np.uint32))
    assert np.array_equal(h.smooth(raw.x).view(np.uint16), o.x_hat.view(np.uint16))
    assert np.array_equal(h.l1t.T.view(np.uint16), o.l1.view(np.uint16))
    assert np.array_equal(h.l2.view(np.uint16), o.l2.view(np.uint16))
    assert np.array_equal(h.r_t.T.view(np.uint32), o.res.view(np.uint32))


@pytest.mark.parametrize("ra", [16, 32, 8])
def test_product_lora_equals_oracle_lora(ra):
    from bit_w4a4_quantized_amd.prepare import attach_lora
    shape = LayerShape("a", 128, 256, 256, 32, "int4", 1000, 8)
    raw = draw_layer(shape)
    h = prepare_host(raw.x, raw.w, raw.b, shape.r)
    g = np.random.default_rng(ra)
    a = (g.standard_normal((256, ra)) * 0.05).astype(np.float16)
    b = (g.standard_normal((ra, 256)) * 0.05).astype(np.float16)
    hl = attach_lora(h, a, b, 0.75)
    l1p, l2p = prep.lora_branch(h.l1t.T, h.l2, h.lam, a, b, 0.75)
    assert np.array_equal(hl.l1t.T.view(np.uint16), l1p.view(np.uint16))
    assert np.array_equal(hl.l2.view(np.uint16), l2p.view(np.uint16))
    assert hl.r_t is h.r_t                   # the residual (and so its codes) is untouched


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_product_gptq_equals_oracle_gptq(fmt):
    from bit_w4a4_quantized_amd.prepare import gptq_residual
    from oracle import gptq
    shape = LayerShape("g", 256, 192, 96, 16, fmt, 21, 6)
    raw = draw_layer(shape)
    h = prepare_host(raw.x, raw.w, raw.b, shape.r)
    x_hat = h.smooth(raw.x)
    codes, scales = gptq_residual(h, x_hat, fmt)
    oc, os_ = gptq.gptq(h.r_t, gptq.hessian(x_hat), fmt)
    assert np.array_equal(codes, oc)
    assert np.array_equal(scales.view(np.uint16), os_.view(np.uint16))
