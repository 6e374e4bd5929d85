"""The neighbouring steps folded into the two kernels, on the GPU.

Kernel A on unsmoothed activations: X_hat = fp16_rne(fp32(x) / lambda) is an exact
definition (IEEE division, one rounding), so codes and scales must match the oracle's
quantization of the oracle's X_hat bit for bit, and all three outputs must equal the plain
Kernel A run on that X_hat.  Kernel B with the MLP glue in its epilogue uses the glue
kernel's own arithmetic, so its output must equal the glue applied to the plain Kernel B
output bit for bit; against the oracle (float64 GELU of the oracle's Y) it is held to the
parity tolerance.  The glue arithmetic itself is pinned over every finite fp16 input.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bit_w4a4_quantized_amd import binding  # noqa: E402
from tests.layers import log, rel_fro, fp16_ulp_diff  # noqa: E402
from tests.layouts import dev_codes, dev_scales  # noqa: E402
from tests.test_gpu_kernels import FMTS, TOL, _gemm_inputs, dev, host, same_bytes  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield
    torch.cuda.synchronize()


def raw_input(seed, M, K):
    """Unsmoothed activations (1% outlier channels x30) and smoothing factors with full fp32
    mantissas, log-uniform in [0.05, 20]."""
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, K)) * 0.7
    x[:, g.choice(K, max(1, K // 100), replace=False)] *= 30.0
    lam = np.exp(g.uniform(np.log(0.05), np.log(20.0), K)).astype(np.float32)
    return x.astype(np.float16), lam


SMOOTH_SHAPES = [  # M, K, r; (2048, 3072, 32): enough row blocks that K is cut into fewer,
    # longer slices than at the sizes above (the smoothing variant must slice K as the plain
    # one does, whatever its row blocks, for T to match bit for bit)
    (1, 64, 0), (3, 128, 16), (17, 192, 32), (130, 320, 32), (257, 256, 64), (300, 128, 48),
    (520, 320, 32), (77, 12288, 16), (300, 2048, 32), (200, 4096, 64), (129, 1024, 48), (2048, 3072, 32),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,r", SMOOTH_SHAPES)
@pytest.mark.parametrize("sliced", [True, False])
def test_quantize_down_smooth_parity(fmt, M, K, r, sliced):
    log(f"quantize_down_smooth {fmt} M={M} K={K} r={r} sliced={sliced}")
    x, lam = raw_input(M * 5 + K + r, M, K)
    l1 = (np.random.default_rng(K + r).standard_normal((K, r)) * 0.3).astype(np.float16)
    x_hat = oracle.prep.smooth_activations(x, lam)
    q, s, stored = oracle.quant.quantize(x_hat, fmt)
    gl = dev(l1.T) if r else None
    xq, xs, t = binding.svdq_quantize_down_smooth(dev(x), dev(lam), gl, fmt, no_workspace=not sliced)
    assert same_bytes(host(xq), dev_codes(stored, fmt))
    assert same_bytes(host(xs), dev_scales(s, fmt))
    pq, ps, pt = binding.svdq_quantize_down(dev(x_hat), gl, fmt, no_workspace=not sliced)
    assert same_bytes(host(xq), host(pq)) and same_bytes(host(xs), host(ps))
    if r:
        assert same_bytes(host(t), host(pt))
        assert rel_fro(host(t), oracle.forward.down_projection(x_hat, l1)) <= TOL


def _partial_round_shape():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles_m = -(-(2 * cus + 8) // 8)
    return 128 * tiles_m - 37, 192, 1024


GELU_SHAPES = [  # M, K, N, r: every Kernel B path (weight streaming at M <= 256 in 32-, 64- and
    # 128-row slabs, tiles, the sub-tile jobs of a last partial round, ragged edges)
    (1, 64, 16, 0), (33, 192, 48, 32), (150, 256, 80, 32), (200, 320, 144, 32), (520, 320, 272, 32),
    (300, 128, 400, 48),
    "partial",
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shape", GELU_SHAPES)
@pytest.mark.parametrize("with_bias", [True, False])
def test_gemm_gelu_smooth_is_glue_of_gemm(fmt, shape, with_bias):
    M, K, N = _partial_round_shape() if shape == "partial" else shape[:3]
    r = 32 if shape == "partial" else shape[3]
    log(f"gemm_w4a4_up_gelu_smooth {fmt} M={M} K={K} N={N} r={r} bias={with_bias}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 3 * M + N + r)
    lam = np.exp(np.random.default_rng(N).uniform(np.log(0.2), np.log(8.0), N)).astype(np.float32)
    args = (dev(dev_codes(xst, fmt)), dev(dev_scales(xs, fmt)), dev(t) if r else None, dev(dev_codes(wst, fmt)),
            dev(dev_scales(ws, fmt)), dev(l2) if r else None, dev(b) if with_bias else None)
    folded = binding.svdq_gemm_w4a4_up_gelu_smooth(*args, dev(lam), K, fmt)
    plain = binding.svdq_gemm_w4a4_up(*args, K, fmt)
    glued = binding.svdq_gelu_tanh_smooth(plain, dev(lam))
    assert same_bytes(host(folded), host(glued))
    ref = oracle.forward.gelu_smooth(oracle.forward.linear(xq, xs, t, wq, ws, l2, b if with_bias else None, fmt), lam)
    assert rel_fro(host(folded), ref) <= TOL


@pytest.mark.parametrize("with_bias", [True, False])
def test_gemm_gelu_smooth_mxfp4_large_tiles(with_bias):
    # the 256 x 256 tile epilogue with the glue folded in (MXFP4, one round of large tiles on 256
    # CUs, ragged edges, padding steps)
    fmt, M, K, N, r = "mxfp4", 4000, 1088, 4000, 32
    log(f"gemm_w4a4_up_gelu_smooth large tiles {fmt} M={M} K={K} N={N} r={r} bias={with_bias}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 5 * M + N)
    lam = np.exp(np.random.default_rng(N + 1).uniform(np.log(0.2), np.log(8.0), N)).astype(np.float32)
    args = (dev(dev_codes(xst, fmt)), dev(dev_scales(xs, fmt)), dev(t), dev(dev_codes(wst, fmt)),
            dev(dev_scales(ws, fmt)), dev(l2), dev(b) if with_bias else None)
    folded = binding.svdq_gemm_w4a4_up_gelu_smooth(*args, dev(lam), K, fmt)
    plain = binding.svdq_gemm_w4a4_up(*args, K, fmt)
    glued = binding.svdq_gelu_tanh_smooth(plain, dev(lam))
    assert same_bytes(host(folded), host(glued))
    ref = oracle.forward.gelu_smooth(oracle.forward.linear(xq, xs, t, wq, ws, l2, b if with_bias else None, fmt), lam)
    assert rel_fro(host(folded), ref) <= TOL


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N,r", [(17, 192, 48, 32), (300, 320, 272, 32), (1, 64, 16, 0)])
def test_linear_folded(fmt, M, K, N, r):
    log(f"linear_folded {fmt} M={M} K={K} N={N} r={r}")
    x, lam_in = raw_input(M + K, M, K)
    x_hat = oracle.prep.smooth_activations(x, lam_in)
    g = np.random.default_rng(M + N)
    l1 = (g.standard_normal((K, r)) * 0.3).astype(np.float16)
    l2 = (g.standard_normal((r, N)) * 0.3).astype(np.float16)
    b = (g.standard_normal(N) * 0.01).astype(np.float16)
    lam_next = np.exp(g.uniform(np.log(0.2), np.log(8.0), N)).astype(np.float32)
    r_t = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    wq, ws = binding.svdq_quantize_weight(dev(r_t), fmt)
    gl1, gl2 = (dev(l1.T), dev(l2)) if r else (None, None)
    plain = binding.svdq_linear(dev(x_hat), gl1, wq, ws, gl2, dev(b), fmt)
    f00 = binding.svdq_linear_folded(dev(x_hat), None, gl1, wq, ws, gl2, dev(b), None, fmt)
    f10 = binding.svdq_linear_folded(dev(x), dev(lam_in), gl1, wq, ws, gl2, dev(b), None, fmt)
    f11 = binding.svdq_linear_folded(dev(x), dev(lam_in), gl1, wq, ws, gl2, dev(b), dev(lam_next), fmt)
    f01 = binding.svdq_linear_folded(dev(x_hat), None, gl1, wq, ws, gl2, dev(b), dev(lam_next), fmt)
    glued = binding.svdq_gelu_tanh_smooth(plain, dev(lam_next))
    assert same_bytes(host(f00), host(plain))
    assert same_bytes(host(f10), host(plain))
    assert same_bytes(host(f11), host(glued))
    assert same_bytes(host(f01), host(glued))


def test_mlp_pair_chain():
    # fc1 with both folds, then fc2 on its output: each stage against the oracle on that
    # stage's own input (the first stage's fp32 summation order may move Y1 by an ulp, so the
    # second stage is checked on the GPU's X_hat2, which the oracle quantizes the same way)
    fmt, M, K1, N1, K2 = "int4_e2m3", 300, 256, 512, 512
    r = 32
    x, lam1 = raw_input(11, M, K1)
    g = np.random.default_rng(12)
    l1a, l2a = (g.standard_normal((K1, r)) * 0.3).astype(np.float16), (g.standard_normal((r, N1)) * 0.3).astype(np.float16)
    l1b, l2b = (g.standard_normal((K2, r)) * 0.3).astype(np.float16), (g.standard_normal((r, 64)) * 0.3).astype(np.float16)
    ba, bb = (g.standard_normal(N1) * 0.01).astype(np.float16), (g.standard_normal(64) * 0.01).astype(np.float16)
    lam2 = np.exp(g.uniform(np.log(0.2), np.log(8.0), N1)).astype(np.float32)
    ra, rb = (g.standard_normal((N1, K1)) * 0.05).astype(np.float32), (g.standard_normal((64, K2)) * 0.05).astype(np.float32)
    wqa, wsa = binding.svdq_quantize_weight(dev(ra), fmt)
    wqb, wsb = binding.svdq_quantize_weight(dev(rb), fmt)
    x2 = binding.svdq_linear_folded(dev(x), dev(lam1), dev(l1a.T), wqa, wsa, dev(l2a), dev(ba), dev(lam2), fmt)
    y = binding.svdq_linear(x2, dev(l1b.T), wqb, wsb, dev(l2b), dev(bb), fmt)
    # stage 1 against the oracle
    xh = oracle.prep.smooth_activations(x, lam1)
    xq, xs, _ = oracle.quant.quantize(xh, fmt)
    wqa_o, wsa_o, _ = oracle.quant.quantize(ra, fmt)
    ref1 = oracle.forward.gelu_smooth(
        oracle.forward.linear(xq, xs, oracle.forward.down_projection(xh, l1a), wqa_o, wsa_o, l2a, ba, fmt), lam2)
    x2h = host(x2)
    assert rel_fro(x2h, ref1) <= TOL
    # stage 2 on the GPU's X_hat2
    xq2, xs2, _ = oracle.quant.quantize(x2h, fmt)
    wqb_o, wsb_o, _ = oracle.quant.quantize(rb, fmt)
    ref2 = oracle.forward.linear(xq2, xs2, oracle.forward.down_projection(x2h, l1b), wqb_o, wsb_o, l2b, bb, fmt)
    assert rel_fro(host(y), ref2) <= TOL


@pytest.mark.parametrize("lam_value", [1.0, 0.37, 7.3])
def test_gelu_glue_every_fp16_value(lam_value):
    # all finite fp16 inputs (both signs, subnormals, the overflow of the denominator for
    # large negative inputs, the fp16 overflow of v / lambda for lambda < 1): within one fp16
    # ulp of the float64 GELU, exactly rounded
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    v = v[np.isfinite(v)]
    C = 64
    n = (v.size // C) * C
    y = np.ascontiguousarray(v[:n].reshape(-1, C))
    lam = np.full(C, lam_value, np.float32)
    out = host(binding.svdq_gelu_tanh_smooth(dev(y), dev(lam)))
    ref = oracle.forward.gelu_smooth(y, lam)
    assert fp16_ulp_diff(out, ref) <= 1
