"""Pins of the VDA-Prep oracle (the linear branch's feature map) to what the
definitions and library routines fix: identity filters reduce it to closed
forms, the separable convolution equals a 3-D correlation computed by
scipy.ndimage, the causal variant equals a brute-force sum, and the
normalised outputs have unit norm."""
import numpy as np
import pytest
import scipy.ndimage as ndi

from oracle import vda_prep as P


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _params(**kw):
    base = dict(grid_h=5, grid_w=6, kernel_h=3, kernel_w=3, taps=5, causal=False, l2_eps=1e-6)
    base.update(kw)
    return P.PrepParams(**base)


def test_silu_closed_form():
    x = np.array([0.0, 1.0, -1.0, 30.0, -30.0])
    want = np.array([0.0, 1.0 / (1.0 + np.exp(-1.0)), -1.0 / (1.0 + np.exp(1.0)), 30.0, 0.0])
    np.testing.assert_allclose(P.silu(x), want, rtol=1e-12, atol=1e-11)


def test_l2_normalize_unit_norm_and_eps():
    x = _rand((7, 16), 1)
    y = P.l2_normalize(x, 0.0)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-13)
    z = P.l2_normalize(np.zeros((2, 4)), 1e-6)
    assert np.all(z == 0.0)
    # eps sits under the root: a vector of norm 1e-3 keeps 1e-3 / sqrt(1e-6 + 1e-6)
    v = np.array([[1e-3, 0.0]])
    np.testing.assert_allclose(P.l2_normalize(v, 1e-6)[0, 0], 1e-3 / np.sqrt(2e-6), rtol=1e-12)


@pytest.mark.parametrize("kh,kw,taps", [(3, 3, 5), (1, 1, 5), (3, 5, 3), (5, 3, 1)])
def test_identity_filters_reduce_to_pointwise(kh, kw, taps):
    p = _params(kernel_h=kh, kernel_w=kw, taps=taps)
    F, d = 4, 8
    L = F * p.grid_h * p.grid_w
    q, k, v = _rand((L, d), 2), _rand((L, d), 3), _rand((L, d), 4)
    w_sp = np.zeros((d, kh, kw))
    w_sp[:, (kh - 1) // 2, (kw - 1) // 2] = 1.0
    w_t = np.zeros((d, taps))
    w_t[:, p.t0] = 1.0
    qo, ko, vo = P.prep_head(q, k, v, w_sp, w_t, p)
    sil = lambda x: x / (1.0 + np.exp(-x))
    nrm = lambda x: x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(qo, nrm(q), rtol=1e-13)
    np.testing.assert_allclose(ko, nrm(sil(k)), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(vo, sil(v), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("kh,kw,taps", [(3, 3, 5), (3, 5, 3), (5, 3, 5), (1, 3, 5)])
def test_short_conv_equals_scipy_3d_correlation(kh, kw, taps):
    p = _params(kernel_h=kh, kernel_w=kw, taps=taps)
    F, d = 7, 5
    x = _rand((F, p.grid_h, p.grid_w, d), 5)
    w_sp = _rand((d, kh, kw), 6)
    w_t = _rand((d, taps), 7)
    got = P.short_conv(x, w_sp, w_t, p)
    for c in range(d):
        ker = w_t[c][:, None, None] * w_sp[c][None, :, :]
        want = ndi.correlate(x[..., c], ker, mode="constant", cval=0.0)
        np.testing.assert_allclose(got[..., c], want, rtol=1e-12, atol=1e-12)


def test_separable_equals_spatial_then_temporal_library():
    p = _params()
    F, d = 9, 3
    x = _rand((F, p.grid_h, p.grid_w, d), 8)
    w_sp = _rand((d, 3, 3), 9)
    w_t = _rand((d, 5), 10)
    got = P.short_conv(x, w_sp, w_t, p)
    for c in range(d):
        sp = np.stack([ndi.correlate(x[f, :, :, c], w_sp[c], mode="constant") for f in range(F)])
        want = ndi.correlate1d(sp, w_t[c], axis=0, mode="constant")
        np.testing.assert_allclose(got[..., c], want, rtol=1e-12, atol=1e-12)


def test_causal_taps_brute_force():
    p = _params(causal=True, grid_h=3, grid_w=4)
    F, d = 6, 2
    x = _rand((F, 3, 4, d), 11)
    w_sp = _rand((d, 3, 3), 12)
    w_t = _rand((d, 5), 13)
    got = P.short_conv(x, w_sp, w_t, p)
    want = np.zeros_like(got)
    for f in range(F):
        for y in range(3):
            for xx in range(4):
                for c in range(d):
                    s = 0.0
                    for tau in range(5):
                        fs = f + tau - 4          # causal: frames f-4 .. f
                        for dy in range(3):
                            for dx in range(3):
                                ys, xs = y + dy - 1, xx + dx - 1
                                if 0 <= fs < F and 0 <= ys < 3 and 0 <= xs < 4:
                                    s += w_t[c, tau] * w_sp[c, dy, dx] * x[fs, ys, xs, c]
                    want[f, y, xx, c] = s
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # frame 0 of a causal filter sees frame 0 only
    x2 = x.copy()
    x2[1:] = 0.0
    np.testing.assert_allclose(P.short_conv(x2, w_sp, w_t, p)[0], got[0], rtol=1e-12, atol=1e-12)


def test_prep_rows_matches_full_head():
    p = _params(grid_h=4, grid_w=5)
    F, d = 8, 6
    L = F * 20
    k, v = _rand((L, d), 14), _rand((L, d), 15)
    w_sp, w_t = _rand((d, 3, 3), 16), _rand((d, 5), 17)
    _, ko, vo = P.prep_head(np.ones((L, d)), k, v, w_sp, w_t, p)
    rows = np.array([0, 1, 19, 20, 77, 80, 139, 159])
    kr, vr = P.prep_rows(k, v, w_sp, w_t, rows, p)
    np.testing.assert_allclose(kr, ko[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(vr, vo[rows], rtol=1e-12, atol=1e-13)


def test_vda_prep_layout_and_unit_norms():
    p = _params(grid_h=2, grid_w=3)
    B, F, H, d = 2, 5, 3, 4
    L = F * 6
    q, k, v = _rand((B, L, H, d), 18), _rand((B, L, H, d), 19), _rand((B, L, H, d), 20)
    w_sp, w_t = _rand((H, d, 3, 3), 21), _rand((H, d, 5), 22)
    qo, ko, vo = P.vda_prep(q, k, v, w_sp, w_t, p)
    assert qo.shape == (B, H, L, d)
    for b in range(B):
        for h in range(H):
            r = P.prep_head(q[b, :, h], k[b, :, h], v[b, :, h], w_sp[h], w_t[h], p)
            np.testing.assert_array_equal(qo[b, h], r[0])
            np.testing.assert_array_equal(ko[b, h], r[1])
            np.testing.assert_array_equal(vo[b, h], r[2])
    nq = np.linalg.norm(qo, axis=-1)
    nk = np.linalg.norm(ko, axis=-1)
    assert np.all(nq < 1.0) and np.all(nq > 1.0 - 1e-5)
    assert np.all(nk <= 1.0) and np.all(nk > 0.99)
