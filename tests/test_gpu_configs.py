"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark times (svdq_linear: Kernel A then Kernel B on one stream).

The oracle computes every output at these sizes (float64 BLAS), so the
comparison is complete, not sampled: codes and scales bit-exact on the full
tensors, Y within 1e-3 relative Frobenius error and within the elementwise fp32
reassociation bound.
"""
import functools

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

import oracle  # noqa: E402
from bit_w4a4_quantized_amd import binding  # noqa: E402
from tests.layers import (log, prepared, raw_layer, reference, rel_fro, within_sum_bound,  # noqa: E402
                          linear_abs_sum, branch_slack, w4a16_bound_terms, gemm_terms)
from tests.layouts import dev_codes, dev_scales  # noqa: E402

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bytes(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def run_layer(P, fmt, x_hat=None, check_codes=True):
    """GPU: weight quantizer, Kernel A, Kernel B and the fused call; oracle: the same layer."""
    x_hat = P.x_hat if x_hat is None else x_hat
    M, K = x_hat.shape
    N = P.res.shape[1]
    r = P.l1.shape[1]
    log(f"GPU {fmt} M={M} K={K} N={N} r={r}")
    ref = reference(P, fmt, x_hat)
    gx = dev(x_hat)
    gl1t = dev(P.l1.T) if r else None
    gl2 = dev(P.l2) if r else None
    gb = dev(P.bias)
    wq, ws = binding.svdq_quantize_weight(dev(P.res.T), fmt)
    if check_codes:
        assert same_bytes(host(wq), dev_codes(ref["wstored"], fmt)), "weight codes"
        assert same_bytes(host(ws), dev_scales(ref["ws"], fmt)), "weight scales"
        xq, xs, t = binding.svdq_quantize_down(gx, gl1t, fmt)
        assert same_bytes(host(xq), dev_codes(ref["xstored"], fmt)), "activation codes"
        assert same_bytes(host(xs), dev_scales(ref["xs"], fmt)), "activation scales"
        if r:
            tg = host(t)
            assert rel_fro(tg, ref["t"]) <= TOL
            ok, worst = within_sum_bound(tg, ref["t"], np.abs(x_hat.astype(np.float64)) @ np.abs(P.l1.astype(np.float64)), K)
            assert ok, worst
        del xq, xs, t
    y = host(binding.svdq_linear(gx, gl1t, wq, ws, gl2, gb, fmt))
    err = rel_fro(y, ref["y"])
    log(f"  rel_fro={err:.3e}")
    assert np.isfinite(y.astype(np.float32)).all()
    assert err <= TOL
    # the fused call rounds its own T: allow for T's own bound through L2
    slack = branch_slack(x_hat, P.l1, ref["t"], P.l2) if r else 0.0
    ok, worst = within_sum_bound(y, ref["y"], linear_abs_sum(ref["xq"], ref["xs"], ref["t"], ref["wq"], ref["ws"],
                                                             P.l2, P.bias, fmt), gemm_terms(fmt, K, r), slack)
    assert ok, worst
    return y, ref, (wq, ws)


def test_c0_tiny_layer():
    run_layer(prepared("c0", 32), "int4")


@pytest.mark.parametrize("fmt", ["int4", "int4_e2m3"])
def test_c1_qkv(fmt):
    run_layer(prepared("c1_qkv", 32), fmt)


def test_c2_fc1_e2m3_container():
    run_layer(prepared("c2_fc1", 32), "int4_e2m3")


def test_c2_mlp_pair():
    P1 = prepared("c2_fc1", 32)
    y1, ref1, _ = run_layer(P1, "int4")
    P2 = prepared("c2_fc2", 32)
    # glue on the oracle's fc1 output: GPU vs oracle
    xg = host(binding.svdq_gelu_tanh_smooth(dev(ref1["y"]), dev(P2.lam)))
    x2_ref = oracle.forward.gelu_smooth(ref1["y"], P2.lam)
    assert rel_fro(xg, x2_ref) <= TOL
    # fc2 on the same smoothed input for both sides: codes bit-exact
    run_layer(P2, "int4", x_hat=x2_ref)
    # the whole chain on the GPU against the oracle's chain (tolerance only)
    y2_ref = reference(P2, "int4", x2_ref)["y"]
    g = binding
    wq2, ws2 = g.svdq_quantize_weight(dev(P2.res.T), "int4")
    wq1, ws1 = g.svdq_quantize_weight(dev(P1.res.T), "int4")
    y1g = g.svdq_linear(dev(P1.x_hat), dev(P1.l1.T), wq1, ws1, dev(P1.l2), dev(P1.bias), "int4")
    x2g = g.svdq_gelu_tanh_smooth(y1g, dev(P2.lam))
    y2g = host(g.svdq_linear(x2g, dev(P2.l1.T), wq2, ws2, dev(P2.l2), dev(P2.bias), "int4"))
    err = rel_fro(y2g, y2_ref)
    log(f"  chained fc1 -> gelu -> fc2 rel_fro={err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt", ["int4", "int4_e2m3"])
@pytest.mark.parametrize("m", [64, 256, 1024])
def test_c3_small_batch(m, fmt):
    # in the 6-bit container M = 64 and 256 run the weight-streaming kernel, whose four waves
    # each walk 12 of the 48 groups through their register ring; M = 1024 runs the tiled kernel
    P = prepared("c2_fc1", 32)
    run_layer(P, fmt, x_hat=np.ascontiguousarray(P.x_hat[:m]))


def test_c3_w4a16_control():
    L = raw_layer("c2_fc1")
    q, s, st = oracle.quant.quantize(L.w.T.astype(np.float32), "int4")
    ref = oracle.forward.w4a16(L.x, q, s, L.b)
    y = host(binding.svdq_gemm_w4a16(dev(L.x), dev(dev_codes(st, "int4")), dev(dev_scales(s, "int4")), dev(L.b)))
    err = rel_fro(y, ref)
    log(f"  w4a16 rel_fro={err:.3e}")
    assert err <= TOL
    ok, worst = within_sum_bound(y, ref, *w4a16_bound_terms(L.x, q, s, L.b))
    assert ok, worst


def test_c4_fp4():
    run_layer(prepared("c2_fc1", 32), "fp4")


def test_c4_int8():
    run_layer(prepared("c2_fc1", 16), "int8")


@pytest.mark.parametrize("fmt", ["int4", "int4_e2m3"])
@pytest.mark.parametrize("name", ["c1_qkv", "c2_fc1"])
def test_unfused_and_bare(name, fmt):
    P = prepared(name, 32)
    log(f"unfused and bare {name} {fmt}")
    ref = reference(P, fmt)
    wq, ws = binding.svdq_quantize_weight(dev(P.res.T), fmt)
    args = (dev(P.x_hat), dev(P.l1.T), wq, ws, dev(P.l2), dev(P.bias), fmt)
    yu = host(binding.svdq_linear_unfused(*args))
    assert rel_fro(yu, ref["y"]) <= TOL
    y0 = host(binding.svdq_linear(dev(P.x_hat), None, wq, ws, None, dev(P.bias), fmt))
    M, N = y0.shape
    ref0 = oracle.forward.linear(ref["xq"], ref["xs"], np.zeros((M, 0), np.float16), ref["wq"], ref["ws"],
                                 np.zeros((0, N), np.float16), P.bias, fmt)
    assert rel_fro(y0, ref0) <= TOL
    ok, worst = within_sum_bound(y0, ref0, linear_abs_sum(ref["xq"], ref["xs"], None, ref["wq"], ref["ws"], None,
                                                          P.bias, fmt), gemm_terms(fmt, P.x_hat.shape[1], 0))
    assert ok, worst


@functools.lru_cache(maxsize=None)
def fc2_input():
    """The oracle's fc2 input: fp16(gelu(Y1) / lambda2) of the oracle's fc1 output."""
    P1, P2 = prepared("c2_fc1", 32), prepared("c2_fc2", 32)
    return oracle.forward.gelu_smooth(reference(P1, "int4")["y"], P2.lam)


def test_c2_fc2_e2m3_container():
    # K = 12288: 192 groups, 64 stages of three in the tiled kernel
    run_layer(prepared("c2_fc2", 32), "int4_e2m3", x_hat=fc2_input())


@pytest.mark.parametrize("name", ["c1_qkv", "c2_fc1", "c2_fc2"])
def test_mxfp4_full_size(name):
    # 256 x 256 tiles (fc2: K = 12288, one round)
    run_layer(prepared(name, 32), "mxfp4", x_hat=fc2_input() if name == "c2_fc2" else None)


def test_c2_mlp_pair_folded():
    # the MLP pair as the benchmark times it, in the 6-bit container: fc1's Kernel A on the raw
    # activations with fc1's smoothing folded in, fc1's Kernel B writing fc2's smoothed input,
    # then fc2
    fmt = "int4_e2m3"
    P1, P2 = prepared("c2_fc1", 32), prepared("c2_fc2", 32)
    L1 = raw_layer("c2_fc1")
    log("GPU folded MLP pair, full size")
    wq1, ws1 = binding.svdq_quantize_weight(dev(P1.res.T), fmt)
    xq, xs, t = binding.svdq_quantize_down_smooth(dev(L1.x), dev(P1.lam), dev(P1.l1.T), fmt)
    _, s_ref, st_ref = oracle.quant.quantize(P1.x_hat, fmt)
    assert same_bytes(host(xq), dev_codes(st_ref, fmt)), "codes of the smoothed activations"
    assert same_bytes(host(xs), dev_scales(s_ref, fmt)), "scales of the smoothed activations"
    _, _, tp = binding.svdq_quantize_down(dev(P1.x_hat), dev(P1.l1.T), fmt)
    assert same_bytes(host(t), host(tp)), "T from the smoothing variant equals T on the smoothed input"
    args = (xq, xs, t, wq1, ws1, dev(P1.l2), dev(P1.bias))
    x2 = binding.svdq_gemm_w4a4_up_gelu_smooth(*args, dev(P2.lam), P1.x_hat.shape[1], fmt)
    glued = binding.svdq_gelu_tanh_smooth(binding.svdq_gemm_w4a4_up(*args, P1.x_hat.shape[1], fmt), dev(P2.lam))
    x2h = host(x2)
    assert same_bytes(x2h, host(glued)), "folded epilogue equals the glue on the plain output"
    err = rel_fro(x2h, fc2_input())
    log(f"  fc2 input rel_fro={err:.3e}")
    assert err <= TOL
    # fc2 on the GPU's own input (the oracle quantizes the same fp16 values)
    run_layer(P2, fmt, x_hat=x2h)


@pytest.mark.parametrize("ra", [16, 32])
def test_lora_full_size(ra):
    # fc1 with a LoRA adapter in the branch (rank 32 + ra = 48 or 64), the residual's codes as
    # they are, in the 6-bit container
    fmt = "int4_e2m3"
    P = prepared("c2_fc1", 32)
    K, N = P.res.shape
    g = np.random.default_rng(5 + ra)
    a = (g.standard_normal((K, ra)) * 0.02).astype(np.float16)
    b = (g.standard_normal((ra, N)) * 0.02).astype(np.float16)
    l1p, l2p = oracle.prep.lora_branch(P.l1, P.l2, P.lam, a, b, 1.0)
    rr = l1p.shape[1]
    log(f"GPU LoRA fc1 r={rr}")
    ref = reference(P, fmt)
    tref = oracle.forward.down_projection(P.x_hat, l1p)
    yref = oracle.forward.linear(ref["xq"], ref["xs"], tref, ref["wq"], ref["ws"], l2p, P.bias, fmt)
    wq, ws = binding.svdq_quantize_weight(dev(P.res.T), fmt)
    y = host(binding.svdq_linear(dev(P.x_hat), dev(l1p.T), wq, ws, dev(l2p), dev(P.bias), fmt))
    err = rel_fro(y, yref)
    log(f"  rel_fro={err:.3e}")
    assert err <= TOL
    slack = branch_slack(P.x_hat, l1p, tref, l2p)
    ok, worst = within_sum_bound(y, yref, linear_abs_sum(ref["xq"], ref["xs"], tref, ref["wq"], ref["ws"], l2p,
                                                         P.bias, fmt), gemm_terms(fmt, K, rr), slack)
    assert ok, worst
