"""GPU parity of every entry point against the CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails.

Bar: codes and scales bit-exact; fp16 outputs within 1e-3 relative Frobenius
error of the oracle (and, where the result is one rounding of a sum, within
one fp16 ulp elementwise); the exact int4 grid bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from bit_w4a4_quantized_amd import binding  # noqa: E402
from tests.layers import log, rel_fro, fp16_ulp_diff, within_sum_bound, linear_abs_sum, w4a16_bound_terms, gemm_terms  # noqa: E402
from tests.layouts import dev_codes, dev_scales  # noqa: E402

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.lib()
    yield
    torch.cuda.synchronize()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def same_bytes(a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


FMTS = ["int4", "int8", "fp4", "int4_e2m3", "mxfp4"]


def canonical(q, s, stored, fmt):
    """The oracle's codes and scales in the exchange layout (its row-major storage)."""
    return stored, s


def assert_canonical(xq, xs, K, fmt, q, s, stored):
    """The device codes and scales, turned into the exchange layout on the GPU, equal the
    oracle's exchange bytes."""
    cc, cs = canonical(q, s, stored, fmt)
    gc, gs = binding.svdq_relayout(xq, xs, K, fmt, to_canonical=True)
    assert same_bytes(host(gc), cc), "codes in the exchange layout"
    assert same_bytes(host(gs), cs), "scales in the exchange layout"


def draw(seed, M, K, N, r, xscale=0.7, rscale=0.05):
    g = np.random.default_rng(seed)
    x_hat = (g.standard_normal((M, K)) * xscale)
    cols = g.choice(K, max(1, K // 100), replace=False)
    x_hat[:, cols] *= 5.0
    x_hat = x_hat.astype(np.float16)
    r_t = (g.standard_normal((N, K)) * rscale).astype(np.float32)
    l1 = (g.standard_normal((K, r)) * 0.3).astype(np.float16)
    l2 = (g.standard_normal((r, N)) * 0.3).astype(np.float16)
    b = (g.standard_normal(N) * 0.01).astype(np.float16)
    return x_hat, r_t, l1, l2, b


SHAPES = [  # M, K, N, r
    (1, 64, 16, 0), (3, 128, 32, 16), (17, 192, 48, 32), (64, 64, 128, 32),
    (130, 320, 272, 32), (257, 256, 144, 64), (300, 128, 400, 48), (128, 256, 256, 32),
    (2100, 128, 4096, 16),  # more 128 x 128 tiles than two workgroups per CU: persistent loop
    (520, 320, 272, 32),    # 128 x 128 tiles, 5 groups: a full and a partial stage of 3
    (200, 320, 144, 32),    # few rows (4 row tiles of 32 per workgroup), 5 groups over 4 waves
]


# Kernel A shapes: the GEMM shapes plus long K (K sliced over many workgroups, several chunks per
# wave) with ragged M, and r = 48 / 64 (32-row blocks)
QD_SHAPES = SHAPES + [(300, 2048, 16, 32), (77, 12288, 16, 16), (200, 4096, 16, 64), (129, 1024, 16, 48)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N,r", QD_SHAPES)
@pytest.mark.parametrize("sliced", [True, False])
def test_quantize_down_parity(fmt, M, K, N, r, sliced):
    log(f"quantize_down {fmt} M={M} K={K} r={r} sliced={sliced} "
        f"workspace={binding.quantize_down_workspace_bytes(M, K, r, fmt)}")
    x_hat, _, l1, _, _ = draw(M * 7 + K + r, M, K, 16, r)
    q, s, stored = oracle.quant.quantize(x_hat, fmt)
    xq, xs, t = binding.svdq_quantize_down(dev(x_hat), dev(l1.T) if r else None, fmt, no_workspace=not sliced)
    assert same_bytes(host(xq), dev_codes(stored, fmt))
    assert same_bytes(host(xs), dev_scales(s, fmt))
    assert_canonical(xq, xs, K, fmt, q, s, stored)
    if r:
        tr = oracle.forward.down_projection(x_hat, l1)
        tg = host(t)
        assert rel_fro(tg, tr) <= TOL
        ok, worst = within_sum_bound(tg, tr, np.abs(x_hat.astype(np.float64)) @ np.abs(l1.astype(np.float64)), K)
        assert ok, worst


def test_quantize_down_deterministic_and_workspace_reuse():
    # the sliced path adds the slices in a fixed order: repeated calls, a reused workspace
    # holding the previous call's partials, and a larger workspace give identical bytes
    M, K, r, fmt = 300, 4096, 32, "int4_e2m3"
    x_hat, _, l1, _, _ = draw(91, M, K, 16, r)
    gx, gl = dev(x_hat), dev(l1.T)
    nb = binding.quantize_down_workspace_bytes(M, K, r, fmt)
    assert nb > 0
    ws = torch.full((nb + 4096,), 0xFF, dtype=torch.uint8, device="cuda")
    ref = [host(v) for v in binding.svdq_quantize_down(gx, gl, fmt, workspace=ws)]
    for _ in range(2):
        got = [host(v) for v in binding.svdq_quantize_down(gx, gl, fmt, workspace=ws)]
        assert all(same_bytes(a, b) for a, b in zip(got, ref))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(16, 64), (48, 192), (272, 320), (1024, 512)])
def test_quantize_weight_parity(fmt, N, K):
    log(f"quantize_weight {fmt} N={N} K={K}")
    g = np.random.default_rng(N + K)
    r_t = (g.standard_normal((N, K)) * 10.0 ** g.integers(-4, 1, (N, 1))).astype(np.float32)
    q, s, stored = oracle.quant.quantize(r_t, fmt)
    wq, ws = binding.svdq_quantize_weight(dev(r_t), fmt)
    assert same_bytes(host(wq), dev_codes(stored, fmt))
    assert same_bytes(host(ws), dev_scales(s, fmt))
    assert_canonical(wq, ws, K, fmt, q, s, stored)


def test_quantizers_subnormal_scales_and_zero_groups():
    # tiny values push fp16 scales into subnormals; a zero group gives scale 0 and codes 0
    g = np.random.default_rng(3)
    x = (g.standard_normal((5, 256)) * 1e-6).astype(np.float16)
    x[:, 64:128] = 0
    for fmt in FMTS:
        q, s, stored = oracle.quant.quantize(x, fmt)
        xq, xs, _ = binding.svdq_quantize_down(dev(x), None, fmt)
        assert same_bytes(host(xq), dev_codes(stored, fmt)), fmt
        assert same_bytes(host(xs), dev_scales(s, fmt)), fmt
        wq, ws = binding.svdq_quantize_weight(dev(x.astype(np.float32)[:, :].repeat(16, axis=0)[:80]), fmt)
        q2, s2, st2 = oracle.quant.quantize(x.astype(np.float32).repeat(16, axis=0)[:80], fmt)
        assert same_bytes(host(wq), dev_codes(st2, fmt)), fmt
        assert same_bytes(host(ws), dev_scales(s2, fmt)), fmt


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,K", [(1, 64), (16, 320), (300, 1024)])
def test_relayout_round_trip(fmt, rows, K):
    # exchange -> device gives exactly what Kernel A writes; device -> exchange gives the
    # oracle's bytes back; both directions on every format (the 6-bit container's fields are
    # converted from and to INT4 nibbles)
    log(f"relayout {fmt} rows={rows} K={K}")
    g = np.random.default_rng(rows + K)
    v = (g.standard_normal((rows, K)) * 10.0 ** g.integers(-3, 2, (rows, 1))).astype(np.float16)
    v[:, :64][0] = 0                         # a zero group: scale 0, codes 0
    q, s, stored = oracle.quant.quantize(v, fmt)
    cc, cs = canonical(q, s, stored, fmt)
    xq, xs, _ = binding.svdq_quantize_down(dev(v), None, fmt)
    dq, ds = binding.svdq_relayout(dev(cc), dev(cs), K, fmt, to_canonical=False)
    assert same_bytes(host(dq), host(xq)) and same_bytes(host(ds), host(xs))
    bc, bs = binding.svdq_relayout(dq, ds, K, fmt, to_canonical=True)
    assert same_bytes(host(bc), cc) and same_bytes(host(bs), cs)


def _gemm_inputs(fmt, M, K, N, r, seed):
    x_hat, r_t, l1, l2, b = draw(seed, M, K, N, r)
    xq, xs, xst = oracle.quant.quantize(x_hat, fmt)
    wq, ws, wst = oracle.quant.quantize(r_t, fmt)
    t = oracle.forward.down_projection(x_hat, l1)
    return x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N,r", SHAPES)
@pytest.mark.parametrize("with_bias", [True, False])
def test_gemm_up_parity(fmt, M, K, N, r, with_bias):
    log(f"gemm_w4a4_up {fmt} M={M} K={K} N={N} r={r} bias={with_bias}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, M + N + K + r)
    bias = b if with_bias else None
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2, bias, fmt)
    y = binding.svdq_gemm_w4a4_up(dev(dev_codes(xst, fmt)), dev(dev_scales(xs, fmt)), dev(t) if r else None, dev(dev_codes(wst, fmt)),
                                  dev(dev_scales(ws, fmt)), dev(l2) if r else None,
                                  dev(bias) if with_bias else None, K, fmt)
    yg = host(y)
    assert np.isfinite(yg.astype(np.float32)).all()
    assert rel_fro(yg, ref) <= TOL
    ok, worst = within_sum_bound(yg, ref, linear_abs_sum(xq, xs, t, wq, ws, l2, bias, fmt), gemm_terms(fmt, K, r))
    assert ok, worst


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("r,with_bias", [(32, True), (0, False), (64, True)])
def test_gemm_partial_last_round(fmt, r, with_bias):
    # Tile counts just above a whole number of persistent rounds (two workgroups per CU): the
    # last few 128 x 128 tiles run as 32 x 32 sub-tile jobs.  Ragged M (last tile 91 rows) and an
    # odd number of K groups.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K = 1024, 192
    tiles_m = -(-(2 * cus + 8) // 8)
    M = 128 * tiles_m - 37
    log(f"gemm_w4a4_up tail round {fmt} M={M} K={K} N={N} r={r} CUs={cus}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 4242 + r)
    bias = b if with_bias else None
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2, bias, fmt)
    y = binding.svdq_gemm_w4a4_up(dev(dev_codes(xst, fmt)), dev(dev_scales(xs, fmt)), dev(t) if r else None,
                                  dev(dev_codes(wst, fmt)), dev(dev_scales(ws, fmt)), dev(l2) if r else None,
                                  dev(bias) if with_bias else None, K, fmt)
    yg = host(y)
    assert np.isfinite(yg.astype(np.float32)).all()
    assert rel_fro(yg, ref) <= TOL
    ok, worst = within_sum_bound(yg, ref, linear_abs_sum(xq, xs, t, wq, ws, l2, bias, fmt), gemm_terms(fmt, K, r))
    assert ok, worst


# Long K at few rows: each wave of the weight-streaming kernels (6-bit container and packed INT4,
# M <= 256) walks K/256 groups through its register ring, and the other formats' K loops run
# many stages, so every ring wraps several times; cases for each row-tile count of the streaming
# kernels (1, 2, 4 rows of 32 tiles per workgroup)
RING_SHAPES = [(17, 1024, 272, 32), (64, 3072, 272, 32), (130, 3072, 272, 32), (256, 1024, 272, 64),
               (64, 1024, 272, 0), (300, 3072, 272, 32),
               # either side of the packed format's switch from 32- to 128-row slabs
               (192, 1024, 272, 32), (193, 1024, 272, 32)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N,r", RING_SHAPES)
def test_gemm_long_k_rings(fmt, M, K, N, r):
    log(f"gemm_w4a4_up long K {fmt} M={M} K={K} N={N} r={r}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 7 * M + K + r)
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2, b, fmt)
    y = binding.svdq_gemm_w4a4_up(dev(dev_codes(xst, fmt)), dev(dev_scales(xs, fmt)), dev(t) if r else None,
                                  dev(dev_codes(wst, fmt)), dev(dev_scales(ws, fmt)), dev(l2) if r else None,
                                  dev(b), K, fmt)
    yg = host(y)
    assert rel_fro(yg, ref) <= TOL
    ok, worst = within_sum_bound(yg, ref, linear_abs_sum(xq, xs, t, wq, ws, l2, b, fmt), gemm_terms(fmt, K, r))
    assert ok, worst


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_partial_last_round_long_k(fmt):
    # the sub-tile jobs of a last partial round at K = 3072 (48 groups): each job's four waves
    # walk 12 groups (6-bit container) or 12 chunks (MXFP4, FP4) through their register rings
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K, r = 1024, 3072, 32
    tiles_m = -(-(2 * cus + 8) // 8)
    M = 128 * tiles_m - 37
    log(f"gemm_w4a4_up tail round, long K {fmt} M={M} K={K} N={N} r={r} CUs={cus}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 4343)
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2, b, fmt)
    y = binding.svdq_gemm_w4a4_up(dev(dev_codes(xst, fmt)), dev(dev_scales(xs, fmt)), dev(t), dev(dev_codes(wst, fmt)),
                                  dev(dev_scales(ws, fmt)), dev(l2), dev(b), K, fmt)
    yg = host(y)
    assert rel_fro(yg, ref) <= TOL
    ok, worst = within_sum_bound(yg, ref, linear_abs_sum(xq, xs, t, wq, ws, l2, b, fmt), gemm_terms(fmt, K, r))
    assert ok, worst


# MXFP4 at sizes where the launch takes 256 x 256 tiles (on 256 CUs, K >= 1024): one round with
# ragged last tile row and column, a one-chunk last step and three padding steps (K = 1088: 17
# chunks in two-chunk steps, rounded up to a multiple of four steps); two tiles per workgroup,
# so the ring runs on into the next tile, with padding (K = 1216) and r = 64; four rounds, the
# last one partial, with a half-empty last tile row, at the smallest K (1024: eight steps); every
# rank (the epilogue's operands load before the last step up to r = 32, at its start above); and
# a shape of the same size at K = 192, which stays on the 128 x 128 tiles
@pytest.mark.parametrize("M,K,N,r,with_bias", [(4000, 1088, 4000, 32, True), (4000, 1088, 4000, 0, False),
                                               (4096, 1216, 8192, 64, True), (4224, 1024, 12288, 32, True),
                                               (4000, 1024, 4000, 16, True), (4000, 1024, 4000, 48, False),
                                               (4000, 192, 4000, 32, True)])
def test_mxfp4_large_tiles(M, K, N, r, with_bias):
    fmt = "mxfp4"
    log(f"gemm_w4a4_up large tiles {fmt} M={M} K={K} N={N} r={r} bias={with_bias}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 9 * M + K + r)
    bias = b if with_bias else None
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2, bias, fmt)
    y = binding.svdq_gemm_w4a4_up(dev(dev_codes(xst, fmt)), dev(dev_scales(xs, fmt)), dev(t) if r else None,
                                  dev(dev_codes(wst, fmt)), dev(dev_scales(ws, fmt)), dev(l2) if r else None,
                                  dev(bias) if with_bias else None, K, fmt)
    yg = host(y)
    assert np.isfinite(yg.astype(np.float32)).all()
    assert rel_fro(yg, ref) <= TOL
    ok, worst = within_sum_bound(yg, ref, linear_abs_sum(xq, xs, t, wq, ws, l2, bias, fmt), gemm_terms(fmt, K, r))
    assert ok, worst


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,K,N,r", [(17, 192, 48, 32), (130, 320, 272, 32), (257, 256, 144, 64), (1, 64, 16, 0)])
def test_linear_end_to_end(fmt, M, K, N, r):
    log(f"linear {fmt} M={M} K={K} N={N} r={r}")
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 99 + M)
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2, b, fmt)
    gw, gs = binding.svdq_quantize_weight(dev(np.ascontiguousarray(_rt(fmt, M, K, N, r))), fmt)
    y = binding.svdq_linear(dev(x_hat), dev(l1.T) if r else None, gw, gs, dev(l2) if r else None, dev(b), fmt)
    assert rel_fro(host(y), ref) <= TOL


@pytest.mark.parametrize("fmt", ["int4_e2m3", "mxfp4"])
def test_prepared_layer_equals_linear(fmt):
    # SvdqLinear: weight side checked once, a workspace kept for the largest M seen; a call on
    # more rows regrows it, a call on fewer reuses it -- every output equals svdq_linear's
    K, N, r = 320, 272, 32
    x_hat, l1, l2, b, _, _, _ = _gemm_inputs(fmt, 300, K, N, r, 77)
    gw, gs = binding.svdq_quantize_weight(dev(_rt(fmt, 300, K, N, r)), fmt)
    layer = binding.SvdqLinear(gw, gs, dev(l1.T), dev(l2), dev(b), K, fmt)
    for M in (17, 300, 130):
        gx = dev(x_hat[:M])
        ref = host(binding.svdq_linear(gx, dev(l1.T), gw, gs, dev(l2), dev(b), fmt))
        assert np.array_equal(host(layer(gx)).view(np.uint16), ref.view(np.uint16))


def _rt(fmt, M, K, N, r):
    return draw(99 + M, M, K, N, r)[1]


def _grid(g, rows, K):
    q = g.integers(-7, 8, (rows, K))
    for gi in range(K // 64):
        q[np.arange(rows), gi * 64 + g.integers(0, 64, rows)] = g.choice([-7, 7], rows)
    return q


@pytest.mark.parametrize("fmt", ["int4", "int4_e2m3"])
@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (33, 192, 48), (200, 320, 144)])
def test_exact_grid_bit_for_bit(M, K, N, fmt):
    g = np.random.default_rng(M + K + N)
    qx, qr = _grid(g, M, K), _grid(g, N, K)
    x_hat = (qx * 2.0 ** -4).astype(np.float16)
    r_t = (qr * 2.0 ** -4).astype(np.float32)
    exact = (qx.astype(object) @ qr.T.astype(object))
    ref = np.array([[float(v) * 2.0 ** -8 for v in row] for row in exact]).astype(np.float16)
    wq, ws = binding.svdq_quantize_weight(dev(r_t), fmt)
    y = binding.svdq_linear(dev(x_hat), None, wq, ws, None, None, fmt)
    assert np.array_equal(host(y).view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("fmt", ["int4", "int4_e2m3"])
def test_unfused_matches_fused(fmt):
    M, K, N, r = 130, 320, 272, 32
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 5)
    ref = oracle.forward.linear(xq, xs, t, wq, ws, l2, b, fmt)
    ws_d = dev(dev_scales(ws, fmt))
    args = (dev(x_hat), dev(l1.T), dev(dev_codes(wst, fmt)), ws_d, dev(l2), dev(b), fmt)
    yu = host(binding.svdq_linear_unfused(*args))
    yf = host(binding.svdq_linear(*args))
    assert rel_fro(yu, ref) <= TOL
    assert rel_fro(yu, yf) <= TOL
    # r = 0: the unfused path is the bare GEMM
    y0 = host(binding.svdq_linear_unfused(dev(x_hat), None, dev(dev_codes(wst, fmt)), ws_d, None, dev(b), fmt))
    ref0 = oracle.forward.linear(xq, xs, np.zeros((M, 0), np.float16), wq, ws, np.zeros((0, N), np.float16), b, fmt)
    assert rel_fro(y0, ref0) <= TOL


@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (130, 320, 272), (300, 256, 144), (2100, 128, 4096)])
def test_w4a16_parity(M, K, N):
    g = np.random.default_rng(M * N)
    x = g.standard_normal((M, K)).astype(np.float16)
    w_t = (g.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = (g.standard_normal(N) * 0.01).astype(np.float16)
    q, s, st = oracle.quant.quantize(w_t, "int4")
    ref = oracle.forward.w4a16(x, q, s, b)
    y = binding.svdq_gemm_w4a16(dev(x), dev(dev_codes(st, "int4")), dev(dev_scales(s, "int4")), dev(b))
    yg = host(y)
    assert rel_fro(yg, ref) <= TOL
    ok, worst = within_sum_bound(yg, ref, *w4a16_bound_terms(x, q, s, b))
    assert ok, worst


@pytest.mark.parametrize("M,C", [(1, 8), (7, 264), (300, 1024)])
def test_gelu_smooth_parity(M, C):
    g = np.random.default_rng(M + C)
    y = (g.standard_normal((M, C)) * 3).astype(np.float16)
    lam = g.uniform(0.3, 8.0, C).astype(np.float32)
    ref = oracle.forward.gelu_smooth(y, lam)
    out = host(binding.svdq_gelu_tanh_smooth(dev(y), dev(lam)))
    assert rel_fro(out, ref) <= TOL
    assert fp16_ulp_diff(out, ref) <= 1


@pytest.mark.parametrize("fmt", ["int4", "int4_e2m3"])
def test_repeat_runs_are_bitwise_identical(fmt):
    M, K, N, r = 257, 256, 144, 32
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 11)
    args = (dev(x_hat), dev(l1.T), dev(dev_codes(wst, fmt)), dev(dev_scales(ws, fmt)), dev(l2), dev(b), fmt)
    first = host(binding.svdq_linear(*args))
    for _ in range(9):
        assert np.array_equal(host(binding.svdq_linear(*args)).view(np.uint16), first.view(np.uint16))


@pytest.mark.parametrize("fmt", FMTS)
def test_outputs_stay_inside_their_buffers(fmt):
    M, K, N, r = 130, 192, 48, 32
    x_hat, l1, l2, b, (xq, xs, xst), (wq, ws, wst), t = _gemm_inputs(fmt, M, K, N, r, 12)
    guard = 4096
    canary = 0x5A

    def guarded(nbytes, dtype, shape):
        buf = torch.full((nbytes + 2 * guard,), canary, dtype=torch.uint8, device="cuda")
        view = buf[guard:guard + nbytes].view(dtype).view(*shape)
        return buf, view

    cb = binding.code_row_bytes(K, fmt)
    bq, gq = guarded(M * cb, torch.uint8, binding.code_shape(M, K, fmt))
    sb = binding.lib().svdq_scale_row_bytes(K, binding.FORMATS[fmt])
    bs, gs = guarded(M * sb, binding.scale_dtype(fmt), binding.scale_shape(M, K, fmt))
    bt, gt = guarded(M * r * 2, torch.float16, (M, r))
    binding.svdq_quantize_down(dev(x_hat), dev(l1.T), fmt, xq=gq, xs=gs, t=gt)
    by, gy = guarded(M * N * 2, torch.float16, (M, N))
    binding.svdq_gemm_w4a4_up(gq, gs, gt, dev(dev_codes(wst, fmt)), dev(dev_scales(ws, fmt)), dev(l2), dev(b), K, fmt, y=gy)
    for buf in (bq, bs, bt, by):
        h = host(buf)
        assert (h[:guard] == canary).all() and (h[-guard:] == canary).all()
    assert same_bytes(host(gq), dev_codes(xst, fmt))


def test_empty_inputs_are_no_ops():
    # zero-size tensors have NULL data pointers: an empty call must still succeed
    K, N = 64, 16
    x = torch.zeros((0, K), dtype=torch.float16, device="cuda")
    xq, xs, t = binding.svdq_quantize_down(x, None, "int4")
    assert tuple(xq.shape) == binding.code_shape(0, K, "int4") == (K // 64, 0, 32)
    wq, ws = binding.svdq_quantize_weight(torch.zeros((N, K), dtype=torch.float32, device="cuda"), "int4")
    y = binding.svdq_linear(x, None, wq, ws, None, None, "int4")
    assert y.shape == (0, N)


def test_mxfp4_ties_saturation_and_signed_zero():
    # values on the E2M1 tie points (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 times the group's
    # scale), above the largest code (6.5, 7.9: saturate to 6), tiny ones (0.1: a negative one
    # must give code +0, not -0), zeros and exact grid values, in both signs; each group's
    # first value 7.5 2^e
    # fixes its scale at 2^e (e = floor(log2 7.5) + e - 2), e different per group
    M, K = 32, 256
    g = np.random.default_rng(9)
    pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 7.9, 0.1, 0.0, 0.5, 1.5, 3.0, 4.0, 6.0])
    x = np.zeros((M, K))
    for m in range(M):
        for grp in range(K // 32):
            e = int(g.integers(-8, 6))
            vals = g.choice(pts, 32) * np.where(g.random(32) < 0.5, -1.0, 1.0)
            vals[0] = 7.5 * (1 if g.random() < 0.5 else -1)
            x[m, grp * 32:(grp + 1) * 32] = vals * 2.0 ** e
    x16 = x.astype(np.float16)
    q, s, stored = oracle.quant.quantize(x16, "mxfp4")
    xq, xs, _ = binding.svdq_quantize_down(dev(x16), None, "mxfp4")
    assert same_bytes(host(xq), dev_codes(stored, "mxfp4"))
    assert same_bytes(host(xs), dev_scales(s, "mxfp4"))
    w32 = x16.astype(np.float32)
    q2, s2, st2 = oracle.quant.quantize(w32, "mxfp4")
    wq, ws = binding.svdq_quantize_weight(dev(w32), "mxfp4")
    assert same_bytes(host(wq), dev_codes(st2, "mxfp4"))
    assert same_bytes(host(ws), dev_scales(s2, "mxfp4"))
    assert set(np.unique(q).tolist()) == set(range(16)) - {8}   # every code but -0 is reached
