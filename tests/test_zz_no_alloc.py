"""svdq_linear_noalloc: the fused layer with its intermediates in the library's static
per-device scratch instead of a caller workspace.  It runs svdq_linear's kernels on the same
plan, so its output must equal svdq_linear's bit for bit -- here on two calls in a row, the
second on a smaller input (the scratch keeps the first call's contents), in the INT4 storage
formats and MXFP4 -- and match the oracle to the parity tolerance.  Shapes beyond the
scratch are refused before anything is enqueued."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bit_w4a4_quantized_amd import binding  # noqa: E402
from tests.layers import log, rel_fro  # noqa: E402
from tests.test_gpu_kernels import TOL, _gemm_inputs, dev, host  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["int4_e2m3", "int4", "mxfp4"])
def test_noalloc_equals_linear_on_two_calls(fmt):
    # a large call (K sliced into several partial sums, many 128 x 128 tiles), then a smaller
    # one with a ragged M: the scratch holds the first call's codes and partials when the
    # second runs
    for M, K, N, r in ((2304, 3072, 2048, 32), (300, 1024, 272, 32)):
        need = binding.linear_workspace_bytes(M, K, r, fmt)
        log(f"noalloc {fmt} M={M} K={K} N={N} r={r} workspace={need}")
        assert 0 < need <= binding.STATIC_SCRATCH_BYTES
        x_hat, l1, l2, b, (xq, xs, _), (wq, ws, _), t = _gemm_inputs(fmt, M, K, N, r, 31 * M + K)
        r_t = np.random.default_rng(M).standard_normal((N, K)).astype(np.float32) * 0.05
        gw, gs = binding.svdq_quantize_weight(dev(r_t), fmt)
        args = (dev(x_hat), dev(l1.T), gw, gs, dev(l2), dev(b), fmt)
        y_ref = host(binding.svdq_linear(*args))
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
        binding.svdq_linear_noalloc(*args, y)
        yg = host(y)
        assert np.array_equal(yg.view(np.uint16), y_ref.view(np.uint16))
        wq_o, ws_o, _ = oracle.quant.quantize(r_t, fmt)
        ref = oracle.forward.linear(xq, xs, t, wq_o, ws_o, l2, b, fmt)
        assert rel_fro(yg, ref) <= TOL


def test_noalloc_refuses_shapes_beyond_its_scratch():
    M, K, N, r, fmt = 8192, 12288, 16, 32, "int4_e2m3"
    assert binding.linear_workspace_bytes(M, K, r, fmt) > binding.STATIC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    wq = torch.zeros(binding.code_shape(N, K, fmt), dtype=torch.uint8, device="cuda")
    ws = torch.zeros(binding.scale_shape(N, K, fmt), dtype=torch.float16, device="cuda")
    l1t = torch.zeros((r, K), dtype=torch.float16, device="cuda")
    l2 = torch.zeros((r, N), dtype=torch.float16, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.float16, device="cuda")
    with pytest.raises(binding.SvdqError) as e:
        binding.svdq_linear_noalloc(x, l1t, wq, ws, l2, None, fmt, y)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())            # nothing was enqueued
