"""A LoRA adapter carried by the 16-bit branch, on the GPU: the residual's device codes are
reused as they are and the kernels run at the grown rank (48 or 64); the layer must match the
oracle's forward with the oracle's grown branch (lora_branch) to the parity tolerance."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bit_w4a4_quantized_amd import binding  # noqa: E402
from bit_w4a4_quantized_amd.prepare import attach_lora, prepare_host, to_device, with_branch  # noqa: E402
from synth import LayerShape, draw_layer  # noqa: E402
from tests.layers import log, rel_fro  # noqa: E402
from tests.test_gpu_kernels import FMTS, TOL, dev, host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("ra", [16, 32])
def test_lora_through_the_branch(fmt, ra):
    M, K, N, r = 300, 320, 272, 32
    log(f"lora {fmt} M={M} K={K} N={N} r={r}+{ra}")
    raw = draw_layer(LayerShape("lora", M, K, N, r, fmt, 77 + ra, 8))
    h = prepare_host(raw.x, raw.w, raw.b, r)
    d = to_device(h, fmt)
    g = np.random.default_rng(ra)
    a = (g.standard_normal((K, ra)) * 0.1).astype(np.float16)
    b = (g.standard_normal((ra, N)) * 0.1).astype(np.float16)
    hl = attach_lora(h, a, b, 0.5)
    dl = with_branch(d, hl)
    assert dl.wq is d.wq and dl.ws is d.ws and dl.r == r + ra
    x_hat = h.smooth(raw.x)
    y = binding.svdq_linear(dev(x_hat), dl.l1t, dl.wq, dl.ws, dl.l2, dl.bias, fmt)
    l1p, l2p = oracle.prep.lora_branch(h.l1t.T, h.l2, h.lam, a, b, 0.5)
    xq, xs, _ = oracle.quant.quantize(x_hat, fmt)
    wq, ws, _ = oracle.quant.quantize(h.r_t, fmt)
    t = oracle.forward.down_projection(x_hat, l1p)
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2p, h.bias, fmt)
    assert rel_fro(host(y), ref) <= TOL
    # the adapter is really there: removing it moves the output by scale X A B (up to the
    # fp16 rounding of the two outputs, a few percent of that difference here)
    y0 = host(binding.svdq_linear(dev(x_hat), d.l1t, d.wq, d.ws, d.l2, d.bias, fmt)).astype(np.float64)
    delta = 0.5 * raw.x.astype(np.float64) @ a.astype(np.float64) @ b.astype(np.float64)
    assert rel_fro(host(y).astype(np.float64) - y0, delta) < 0.05
