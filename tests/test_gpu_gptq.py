"""GPTQ codes of the residual through the unchanged kernels, on the GPU.

svdq_pack_weight puts host-computed codes and scales into Kernel B's layout: with the
round-to-nearest codes it must reproduce svdq_quantize_weight bit for bit.  A layer whose
residual was rounded by GPTQ must match the oracle's forward with the oracle's GPTQ codes to
the parity tolerance, and lower the error against the unquantized layer on the calibration
inputs below the round-to-nearest layer's."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bit_w4a4_quantized_amd import binding  # noqa: E402
from bit_w4a4_quantized_amd.prepare import gptq_residual, prepare_host, to_device, to_device_packed  # noqa: E402
from synth import LayerShape, draw_layer  # noqa: E402
from tests.layers import log, rel_fro  # noqa: E402
from tests.test_gpu_kernels import TOL, dev, host, same_bytes  # noqa: E402

INT_FMTS = ["int4", "int4_e2m3", "int8"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", INT_FMTS)
@pytest.mark.parametrize("N,K", [(16, 64), (48, 192), (272, 320)])
def test_pack_round_trips_round_to_nearest(fmt, N, K):
    log(f"pack_weight {fmt} N={N} K={K}")
    g = np.random.default_rng(N + K)
    r_t = (g.standard_normal((N, K)) * 10.0 ** g.integers(-4, 1, (N, 1))).astype(np.float32)
    q, s = oracle.quant.quantize_int(r_t, 127 if fmt == "int8" else 7, 64)
    pq, ps = binding.svdq_pack_weight(dev(q), dev(s), fmt)
    wq, ws = binding.svdq_quantize_weight(dev(r_t), fmt)
    assert same_bytes(host(pq), host(wq)) and same_bytes(host(ps), host(ws))


@pytest.mark.parametrize("fmt", INT_FMTS)
def test_gptq_layer(fmt):
    M, K, N, r = 512, 256, 144, 32
    log(f"gptq layer {fmt} M={M} K={K} N={N} r={r}")
    raw = draw_layer(LayerShape("gptq", M, K, N, r, fmt, 31, 8))
    # correlated input channels (as real activations have; with independent channels 2 X^T X
    # is nearly diagonal and GPTQ reduces to round-to-nearest)
    mix = np.eye(K) + np.random.default_rng(5).standard_normal((K, K)) * (0.5 / np.sqrt(K))
    raw.x = (raw.x.astype(np.float64) @ mix).astype(np.float16)
    h = prepare_host(raw.x, raw.w, raw.b, r)
    x_hat = h.smooth(raw.x)
    codes, scales = gptq_residual(h, x_hat, fmt)
    d = to_device_packed(h, fmt, codes, scales)
    y = host(binding.svdq_linear(dev(x_hat), d.l1t, d.wq, d.ws, d.l2, d.bias, fmt))
    oc, os_ = oracle.gptq.gptq(h.r_t, oracle.gptq.hessian(x_hat), fmt)
    xq, xs, _ = oracle.quant.quantize(x_hat, fmt)
    ref = oracle.forward.linear(xq, xs, oracle.forward.down_projection(x_hat, h.l1t.T), oc, os_, h.l2, h.bias, fmt)
    assert rel_fro(y, ref) <= TOL
    # against the unquantized layer X W + b on the calibration inputs
    exact = raw.x.astype(np.float64) @ raw.w.astype(np.float64) + raw.b.astype(np.float64)
    d_rtn = to_device(h, fmt)
    y_rtn = host(binding.svdq_linear(dev(x_hat), d_rtn.l1t, d_rtn.wq, d_rtn.ws, d_rtn.l2, d_rtn.bias, fmt))
    e_gptq, e_rtn = rel_fro(y.astype(np.float64), exact), rel_fro(y_rtn.astype(np.float64), exact)
    log(f"  error vs unquantized: gptq {e_gptq:.4e}, round-to-nearest {e_rtn:.4e}")
    assert e_gptq < e_rtn
