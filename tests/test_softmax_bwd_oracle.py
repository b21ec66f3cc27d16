"""Pins of the Softmax-branch backward oracle: torch autograd (fp64) through a
dense token-masked attention with the gate (a library route unrelated to the
oracle's per-frame formulas), central finite differences on a tiny case, and
two identities every correct gradient obeys: the value gradients sum to the
output gradients (each softmax row sums to one) and, where every query sees
every key, the key gradients sum to zero (a common shift of all keys leaves
every softmax row unchanged)."""
import math

import numpy as np
import pytest
import torch

from oracle import softmax_bwd as SB
from oracle import vdn_oracle as O


def _case(F, N, d, seed):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((F, N, d)) for _ in range(4))
    g = rng.random((F, N))
    return q, k, v, g, do


def _torch_grads(q, k, v, g, do, p):
    F, N, d = q.shape
    mask = np.repeat(np.repeat(O.visibility(F, p).astype(bool), N, 0), N, 1)
    tq, tk, tv, tg = (torch.tensor(x.reshape(F * N, -1) if x.ndim == 3 else x.reshape(F * N),
                                   dtype=torch.float64, requires_grad=True) for x in (q, k, v, g))
    scale = 1.0 / math.sqrt(d) if p.softmax_scale is None else p.softmax_scale
    s = (tq @ tk.T) * scale
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    out = tg[:, None] * (torch.softmax(s, dim=1) @ tv)
    out.backward(torch.from_numpy(do.reshape(F * N, d)))
    return [x.grad.numpy() for x in (tq, tk, tv, tg)]


@pytest.mark.parametrize("F,N,d,anchors,cf", [(20, 3, 8, True, 5), (35, 2, 4, True, 5), (12, 3, 6, False, 3),
                                              (7, 4, 8, True, 5)])
def test_matches_torch_autograd_dense_masked(F, N, d, anchors, cf):
    p = O.Params(anchors=anchors, chunk_frames=cf)
    q, k, v, g, do = _case(F, N, d, F * 10 + N)
    dq, dk, dv, dg = SB.softmax_branch_bwd(q, k, v, g, do, p)
    tq, tk, tv, tg = _torch_grads(q, k, v, g, do, p)
    np.testing.assert_allclose(dq.reshape(F * N, d), tq, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk.reshape(F * N, d), tk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv.reshape(F * N, d), tv, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dg.reshape(F * N), tg, rtol=1e-10, atol=1e-12)


def test_central_finite_differences():
    F, N, d = 10, 2, 3
    p = O.Params()
    q, k, v, g, do = _case(F, N, d, 5)

    def loss(q_, k_, v_, g_):
        _, Oh, _ = O.softmax_branch(q_, k_, v_, g_, p)
        return float(np.sum(Oh * do))

    dq, dk, dv, dg = SB.softmax_branch_bwd(q, k, v, g, do, p)
    rng = np.random.default_rng(0)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("g", g, dg)):
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = dict(q_=q, k_=k, v_=v, g_=g)
            args_m = dict(q_=q, k_=k, v_=v, g_=g)
            args_p[name + "_"] = xp
            args_m[name + "_"] = xm
            fd = (loss(**args_p) - loss(**args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, grad[idx])


def test_value_gradients_sum_to_output_gradients():
    F, N, d = 25, 3, 4
    q, k, v, g, do = _case(F, N, d, 9)
    _, _, dv, _ = SB.softmax_branch_bwd(q, k, v, g, do)
    np.testing.assert_allclose(dv.sum(axis=(0, 1)), (g[..., None] * do).sum(axis=(0, 1)), rtol=1e-12)


def test_key_gradients_sum_to_zero_when_dense():
    # F <= 10 frames: every query frame sees every key frame
    F, N, d = 10, 3, 5
    q, k, v, g, do = _case(F, N, d, 11)
    _, dk, _, _ = SB.softmax_branch_bwd(q, k, v, g, do)
    assert np.abs(dk.sum(axis=(0, 1))).max() < 1e-11 * np.abs(dk).max() * F * N


def test_zero_gate_gives_zero_input_gradients():
    F, N, d = 20, 2, 4
    q, k, v, g, do = _case(F, N, d, 13)
    dq, dk, dv, dg = SB.softmax_branch_bwd(q, k, v, np.zeros_like(g), do)
    assert not dq.any() and not dk.any() and not dv.any()
    _, Oh, _ = O.softmax_branch(q, k, v, np.ones_like(g))
    np.testing.assert_allclose(dg, np.sum(Oh * do, axis=-1), rtol=1e-12)


def test_rows_evaluation_matches_full():
    F, N, d = 25, 3, 4
    p = O.Params()
    q, k, v, g, do = _case(F, N, d, 17)
    dq, dk, dv, _ = SB.softmax_branch_bwd(q, k, v, g, do, p)
    L = F * N
    fl = lambda x: x.reshape(L, -1)
    qrows = np.array([0, 1, 7, 40, 73, 74])
    for kframe in (0, 7, 24):
        krows = kframe * N + np.array([0, 2])
        rq, rk, rv = SB.softmax_bwd_rows(fl(q), fl(k), fl(v), g.reshape(L), fl(do), F, qrows, kframe,
                                         krows, p)
        np.testing.assert_allclose(rq, fl(dq)[qrows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rk, fl(dk)[krows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rv, fl(dv)[krows], rtol=1e-10, atol=1e-12)


# ---- the text-keys option: the T text tokens are keys of every query ----

def _torch_grads_text(q, k, v, g, do, kt, vt, p):
    F, N, d = q.shape
    T = kt.shape[0]
    vis = np.repeat(np.repeat(O.visibility(F, p).astype(bool), N, 0), N, 1)
    mask = np.concatenate([vis, np.ones((F * N, T), bool)], axis=1)
    tq, tk, tv, tg = (torch.tensor(x.reshape(F * N, -1) if x.ndim == 3 else x.reshape(F * N),
                                   dtype=torch.float64, requires_grad=True) for x in (q, k, v, g))
    tkt, tvt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (kt, vt))
    scale = 1.0 / math.sqrt(d) if p.softmax_scale is None else p.softmax_scale
    s = (tq @ torch.cat([tk, tkt]).T) * scale
    s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    out = tg[:, None] * (torch.softmax(s, dim=1) @ torch.cat([tv, tvt]))
    out.backward(torch.from_numpy(do.reshape(F * N, d)))
    return [x.grad.numpy() for x in (tq, tk, tv, tg, tkt, tvt)]


@pytest.mark.parametrize("F,N,d,T,anchors", [(20, 3, 8, 5, True), (12, 2, 4, 3, False), (7, 4, 6, 1, True)])
def test_text_keys_match_torch_autograd(F, N, d, T, anchors):
    p = O.Params(anchors=anchors, text_softmax=True)
    q, k, v, g, do = _case(F, N, d, F * 7 + T)
    rng = np.random.default_rng(T)
    kt, vt = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    got = SB.softmax_branch_bwd(q, k, v, g, do, p, K_text=kt, V_text=vt)
    want = _torch_grads_text(q, k, v, g, do, kt, vt, p)
    shapes = [(F * N, d)] * 3 + [(F * N,), (T, d), (T, d)]
    for a, b, sh in zip(got, want, shapes):
        np.testing.assert_allclose(a.reshape(sh), b, rtol=1e-10, atol=1e-12)


def test_text_keys_value_gradients_sum_to_output_gradients():
    F, N, d, T = 25, 3, 4, 6
    p = O.Params(text_softmax=True)
    q, k, v, g, do = _case(F, N, d, 19)
    rng = np.random.default_rng(2)
    _, _, dv, _, _, dvt = SB.softmax_branch_bwd(q, k, v, g, do, p, K_text=rng.standard_normal((T, d)),
                                                V_text=rng.standard_normal((T, d)))
    np.testing.assert_allclose(dv.sum(axis=(0, 1)) + dvt.sum(axis=0),
                               (g[..., None] * do).sum(axis=(0, 1)), rtol=1e-12)


def test_text_keys_rows_evaluation_matches_full():
    F, N, d, T = 25, 3, 4, 4
    p = O.Params(text_softmax=True)
    q, k, v, g, do = _case(F, N, d, 23)
    rng = np.random.default_rng(3)
    kt, vt = rng.standard_normal((T, d)), rng.standard_normal((T, d))
    dq, dk, dv, _, _, _ = SB.softmax_branch_bwd(q, k, v, g, do, p, K_text=kt, V_text=vt)
    L = F * N
    fl = lambda x: x.reshape(L, -1)
    qrows = np.array([0, 5, 40, 74])
    for kframe in (0, 12):
        krows = kframe * N + np.array([1, 2])
        rq, rk, rv = SB.softmax_bwd_rows(fl(q), fl(k), fl(v), g.reshape(L), fl(do), F, qrows, kframe,
                                         krows, p, K_text=kt, V_text=vt)
        np.testing.assert_allclose(rq, fl(dq)[qrows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rk, fl(dk)[krows], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(rv, fl(dv)[krows], rtol=1e-10, atol=1e-12)
