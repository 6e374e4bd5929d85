"""The fused layer under HIP graph capture, the use the allocation-free entry point is for.

svdq_linear (caller workspace) and svdq_linear_noalloc (the library's static scratch) are
captured on a side stream and the graph is replayed several times, with the program's own eager
work and synchronizations between replays and new activations copied into the captured input
buffer before some of them: every replay's output must equal the eager call's on the same
inputs, bit for bit (same kernels, same plan), and the eager output must match the oracle.
Shapes: a tiled one with K sliced in Kernel A and a partial last round in Kernel B, and a
few-token one (weight-streaming Kernel B)."""
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


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


@pytest.mark.parametrize("noalloc", [False, True])
@pytest.mark.parametrize("fmt", ["int4_e2m3", "mxfp4"])
@pytest.mark.parametrize("M,K,N,r", [(300, 1024, 272, 32), (64, 1024, 272, 32)])
def test_layer_graph_replays_equal_eager(M, K, N, r, fmt, noalloc):
    log(f"graph {'noalloc' if noalloc else 'linear'} {fmt} M={M} K={K} N={N} r={r}")
    x_hat, l1, l2, b, (xq, xs, _), _, t = _gemm_inputs(fmt, M, K, N, r, 17 * M + K + (7 if noalloc else 0))
    r_t = np.random.default_rng(M + K).standard_normal((N, K)).astype(np.float32) * 0.05
    gw, gs = binding.svdq_quantize_weight(dev(r_t), fmt)
    l1t, l2d, bd = dev(l1.T), dev(l2), dev(b)
    x_in = dev(x_hat)                                    # the captured input buffer
    y_out = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws = None if noalloc else torch.empty(binding.linear_workspace_bytes(M, K, r, fmt), dtype=torch.uint8,
                                          device="cuda")

    def layer(x, y, stream=None):
        if noalloc:
            return binding.svdq_linear_noalloc(x, l1t, gw, gs, l2d, bd, fmt, y, stream=stream)
        return binding.svdq_linear(x, l1t, gw, gs, l2d, bd, fmt, workspace=ws, y=y, stream=stream)

    # eager outputs for two activation sets (the second: another seed, same shape)
    x2 = dev((np.random.default_rng(M * 3 + 1).standard_normal((M, K)) * 0.7).astype(np.float16))
    y1 = host(layer(x_in, torch.empty_like(y_out)))
    y2 = host(layer(x2, torch.empty_like(y_out)))
    wq_o, ws_o, _ = oracle.quant.quantize(r_t, fmt)
    assert rel_fro(y1, oracle.forward.linear(xq, xs, t, wq_o, ws_o, l2, b, fmt)) <= TOL

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        layer(x_in, y_out, stream=side.cuda_stream)
    torch.cuda.synchronize()
    x1 = dev(x_hat)
    for rep, (src, want) in enumerate([(None, y1), (None, y1), (x2, y2), (x1, y1), (x2, y2)]):
        if src is not None:
            x_in.copy_(src)                              # new activations in the captured buffer
        y_out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = host(y_out)
        assert np.array_equal(_bits(got), _bits(want)), f"replay {rep}"
        # the program's own eager work between replays (same library, other buffers)
        layer(x2 if rep % 2 == 0 else dev(x_hat), torch.empty_like(y_out))
        torch.cuda.synchronize()
