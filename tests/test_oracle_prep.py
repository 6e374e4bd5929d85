"""Pins of the oracle's offline setup: smoothing closed forms, Eckart-Young, library SVD cross-check."""
import numpy as np
import pytest
import scipy.linalg

from oracle import prep
from synth import draw_layer, LayerShape


def _small_layer(seed=7, M=96, K=128, N=80, k=6):
    return draw_layer(LayerShape("t", M, K, N, 16, "int4", seed, k))


def test_smoothing_balances_channel_maxima():
    L = _small_layer()
    lam = prep.smoothing_factors(L.x, L.w)
    mx = np.abs(L.x.astype(np.float64)).max(axis=0)
    mw = np.abs(L.w.astype(np.float64)).max(axis=1)
    target = np.sqrt(mx * mw)
    xh = prep.smooth_activations(L.x, lam)
    wh = prep.smooth_weight(L.w, lam)
    # max|X_hat_j| = mx/lambda and max|W_hat_j| = lambda*mw both equal sqrt(mx*mw)
    # up to lambda's fp32 rounding (2^-24 relative, twice) and X_hat's fp16 rounding (2^-11)
    assert np.allclose(np.abs(xh.astype(np.float64)).max(axis=0), target, rtol=2 ** -11 + 1e-6)
    assert np.allclose(np.abs(wh).max(axis=1), target, rtol=1e-6)


def test_smoothing_preserves_product():
    L = _small_layer()
    lam = prep.smoothing_factors(L.x, L.w)
    xh = prep.smooth_activations(L.x, lam).astype(np.float64)
    wh = prep.smooth_weight(L.w, lam)
    ref = L.x.astype(np.float64) @ L.w.astype(np.float64)
    # the only difference is X_hat's rounding: |X_hat - X/lambda| <= 2^-11 |X/lambda| elementwise
    bound = (np.abs(L.x.astype(np.float64) / lam) * 2.0 ** -11) @ np.abs(wh)
    assert (np.abs(xh @ wh - ref) <= bound * (1 + 1e-9) + 1e-12).all()


def test_smoothing_zero_channels_get_unit_factor():
    x = np.ones((4, 3), np.float16)
    x[:, 1] = 0
    w = np.ones((3, 2), np.float16)
    w[2] = 0
    lam = prep.smoothing_factors(x, w)
    assert lam[1] == 1 and lam[2] == 1 and lam[0] == 1


def test_eckart_young_identity():
    L = _small_layer()
    lam = prep.smoothing_factors(L.x, L.w)
    wh = prep.smooth_weight(L.w, lam)
    u, s, vt = np.linalg.svd(wh, full_matrices=False)
    for r in (1, 4, 16):
        approx = (u[:, :r] * s[:r]) @ vt[:r]
        assert np.isclose(np.linalg.norm(wh - approx) ** 2, np.sum(s[r:] ** 2), rtol=1e-9)
        # the oracle's residual is taken against fp16 factors: it is close to, and never below, the optimum
        l1, l2, res, sig = prep.low_rank(wh, r)
        opt = np.sqrt(np.sum(sig[r:] ** 2))
        got = np.linalg.norm(res.astype(np.float64))
        assert got >= opt * (1 - 1e-6)
        assert got <= opt * 1.01 + 1e-3 * np.linalg.norm(wh) * 2 ** -10


@pytest.mark.parametrize("shape,r", [((6, 5), 1), ((6, 5), 2), ((8, 8), 3), ((7, 4), 2)])
def test_eckart_young_search_tiny(shape, r):
    """No rank-r matrix found by random subspace projection or ALS beats the truncated SVD."""
    g = np.random.default_rng(sum(shape) * 10 + r)
    w = g.standard_normal(shape)
    l1, l2, res, sig = prep.low_rank(w, r)
    best = np.sqrt(np.sum(sig[r:] ** 2))
    K, N = shape
    for _ in range(300):
        p, _ = np.linalg.qr(g.standard_normal((N, r)))
        assert np.linalg.norm(w - w @ p @ p.T) >= best * (1 - 1e-12)
        q, _ = np.linalg.qr(g.standard_normal((K, r)))
        assert np.linalg.norm(w - q @ q.T @ w) >= best * (1 - 1e-12)
    for _ in range(20):
        a = g.standard_normal((K, r))
        for _ in range(50):       # alternating least squares from a random start
            b = np.linalg.lstsq(a, w, rcond=None)[0]
            a = np.linalg.lstsq(b.T, w.T, rcond=None)[0].T
        assert np.linalg.norm(w - a @ b) >= best * (1 - 1e-9)
    # the stored fp16 factors reproduce the optimum up to their rounding
    assert np.isclose(np.linalg.norm(res.astype(np.float64)), best, rtol=1e-2, atol=1e-3 * np.linalg.norm(w))


def test_svd_matches_scipy_gesvd_product():
    L = _small_layer(seed=11)
    lam = prep.smoothing_factors(L.x, L.w)
    wh = prep.smooth_weight(L.w, lam)
    l1, l2, res, sig = prep.low_rank(wh, 16)
    u, s, vt = scipy.linalg.svd(wh, full_matrices=False, lapack_driver="gesvd")
    ref = (u[:, :16] * s[:16]) @ vt[:16]
    ours = l1.astype(np.float64) @ l2.astype(np.float64)
    assert np.linalg.norm(ours - ref) <= 2 ** -10 * np.linalg.norm(ref)
    assert np.allclose(sig, s, rtol=1e-10)


def test_residual_definition_and_rank_zero():
    L = _small_layer(seed=3)
    lam = prep.smoothing_factors(L.x, L.w)
    wh = prep.smooth_weight(L.w, lam)
    l1, l2, res, _ = prep.low_rank(wh, 8)
    assert l1.dtype == np.float16 and l2.dtype == np.float16 and res.dtype == np.float32
    assert np.allclose(res.astype(np.float64), wh - l1.astype(np.float64) @ l2.astype(np.float64), rtol=0, atol=np.abs(wh).max() * 2 ** -23)
    l1, l2, res0, _ = prep.low_rank(wh, 0)
    assert l1.shape == (wh.shape[0], 0) and np.array_equal(res0, wh.astype(np.float32))


def test_planted_spectrum_is_steep():
    """Diagnostic of the workload: with a planted rank-k part the k-th gap is large (cf. the spectra the
    reading note describes in its section "Key results", Figure 5)."""
    L = _small_layer(seed=5, K=128, N=128, k=6)
    s = np.linalg.svd(L.w.astype(np.float64), compute_uv=False)
    assert s[5] / s[6] > 3.0
    assert s[6] / s[40] < 2.0


@pytest.mark.parametrize("r,ra", [(32, 16), (32, 32), (16, 8), (0, 16)])
def test_lora_branch_adds_the_adapter_exactly(r, ra):
    # with power-of-two factors and scale and fp16-exact adapter entries, every product is
    # exact, so the grown branch must reproduce X_hat L1 L2 + scale X A B exactly (X = X_hat
    # diag(lambda)); a missing, inverted or misplaced lambda, a transposed factor or a lost
    # scale changes the sum
    g = np.random.default_rng(r + ra)
    M, K, N = 24, 64, 40
    lam = 2.0 ** g.integers(-3, 4, K).astype(np.float64)
    x_hat = (g.integers(-64, 65, (M, K)) / 32.0).astype(np.float16)
    x = x_hat.astype(np.float64) * lam[None, :]
    l1 = (g.integers(-64, 65, (K, r)) / 64.0).astype(np.float16)
    l2 = (g.integers(-64, 65, (r, N)) / 64.0).astype(np.float16)
    a = (g.integers(-32, 33, (K, ra)) / 64.0).astype(np.float16)
    b = (g.integers(-32, 33, (ra, N)) / 64.0).astype(np.float16)
    scale = 0.5
    l1p, l2p = prep.lora_branch(l1, l2, lam.astype(np.float32), a, b, scale)
    assert l1p.shape == (K, -(-(r + ra) // 16) * 16) and l2p.shape == (l1p.shape[1], N)
    assert not l1p[:, r + ra:].any() and not l2p[r + ra:].any()
    got = x_hat.astype(np.float64) @ l1p.astype(np.float64) @ l2p.astype(np.float64)
    want = x_hat.astype(np.float64) @ l1.astype(np.float64) @ l2.astype(np.float64) \
        + scale * (x @ a.astype(np.float64) @ b.astype(np.float64))
    assert np.array_equal(got, want)
