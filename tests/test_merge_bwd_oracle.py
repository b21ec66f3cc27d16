"""Pins of the merge-backward oracle: central finite differences of the
forward merge oracle (vdn_oracle.merge, [B, L, H, dv] heads-concatenated
layout, a different code path) on non-square shapes, so a transposed or
swapped operand cannot pass; the bilinearity identity <dout, out> =
<dOhat_s, Ohat_s> + <dOhat_l, Ohat_l> = <dW_s, W_s> + <dW_l, W_l>; and the
identity projections."""
import numpy as np

from oracle import merge_bwd as MB
from oracle import vdn_oracle as O


def _case(B=2, L=5, H=3, dv=2, D=7, seed=0):
    rng = np.random.default_rng(seed)
    Os, Ol = rng.standard_normal((B, L, H, dv)), rng.standard_normal((B, L, H, dv))
    Ws, Wl = rng.standard_normal((H * dv, D)), rng.standard_normal((H * dv, D))
    dout = rng.standard_normal((B, L, D))
    return Os, Ol, Ws, Wl, dout


def _flat(x):
    return x.reshape(-1, x.shape[-2] * x.shape[-1]) if x.ndim == 4 else x.reshape(-1, x.shape[-1])


def test_central_finite_differences():
    Os, Ol, Ws, Wl, dout = _case()
    dOs, dOl, dWs, dWl = MB.merge_bwd(_flat(Os), _flat(Ol), Ws, Wl, _flat(dout))
    loss = lambda a, b, c, d: float(np.sum(O.merge(a, b, c, d) * dout))
    rng = np.random.default_rng(1)
    h = 1e-6
    for name, x, g, fix in (("Os", Os, dOs, lambda v: (v, Ol, Ws, Wl)), ("Ol", Ol, dOl, lambda v: (Os, v, Ws, Wl)),
                            ("Ws", Ws, dWs, lambda v: (Os, Ol, v, Wl)), ("Wl", Wl, dWl, lambda v: (Os, Ol, Ws, v))):
        gf = g.reshape(x.shape)
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            fd = (loss(*fix(xp)) - loss(*fix(xm))) / (2 * h)
            assert abs(fd - gf[idx]) <= 1e-7 * max(1.0, abs(fd)), (name, idx, fd, gf[idx])


def test_bilinearity_identity():
    Os, Ol, Ws, Wl, dout = _case(B=1, L=11, H=4, dv=3, D=5, seed=2)
    dOs, dOl, dWs, dWl = MB.merge_bwd(_flat(Os), _flat(Ol), Ws, Wl, _flat(dout))
    total = float(np.sum(O.merge(Os, Ol, Ws, Wl) * dout))
    np.testing.assert_allclose(np.sum(dOs * _flat(Os)) + np.sum(dOl * _flat(Ol)), total, rtol=1e-12)
    np.testing.assert_allclose(np.sum(dWs * Ws) + np.sum(dWl * Wl), total, rtol=1e-12)


def test_identity_projections():
    Os, Ol, _, _, _ = _case()
    dout = np.random.default_rng(3).standard_normal(Os.shape)
    dOs, dOl, dWs, dWl = MB.merge_bwd(_flat(Os), _flat(Ol), None, None, _flat(dout))
    np.testing.assert_array_equal(dOs, _flat(dout))
    np.testing.assert_array_equal(dOl, _flat(dout))
    assert dWs is None and dWl is None
