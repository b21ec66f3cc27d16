"""Pins of the oracle's text-aware Softmax option (text keys inside the
Softmax branch, always visible).

Page "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation", method, bidirectional linear attention: the prompt is summarised
into the state that starts both scans, and the text also stays directly
visible to the Softmax branch.  Reading: the T text keys join every video
query's one softmax.  Each pin takes a route other than the oracle's own
(frame list + concatenation): a dense token mask through torch SDPA, a
closed form, the log-sum-exp split of one softmax into two key sets
(scipy), brute force on the dominant key, and invariance of everything the
option must not touch.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

from oracle import vdn_oracle as O

TEXT = O.Params(text_softmax=True)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _dense_mask(F, N, T, p):
    fm = O.visibility(F, p).astype(bool)
    tok = np.repeat(np.repeat(fm, N, axis=0), N, axis=1)
    return np.concatenate([tok, np.ones((F * N, T), bool)], axis=1)


@pytest.mark.parametrize("F,N,T,d", [(20, 4, 3, 8), (35, 3, 16, 16), (7, 5, 1, 4), (10, 2, 9, 8)])
def test_text_softmax_equals_dense_masked_sdpa(F, N, T, d):
    L = F * N
    q, k, v = _rand((L, d), F), _rand((L, d), F + 1), _rand((L, d), F + 2)
    kt, vt = _rand((T, d), F + 3), _rand((T, d), F + 4)
    g = np.random.default_rng(5).random(L)
    O_s, Ohat, lse = O.softmax_branch(q.reshape(F, N, d), k.reshape(F, N, d), v.reshape(F, N, d),
                                      g.reshape(F, N), TEXT, kt, vt)
    mask = _dense_mask(F, N, T, TEXT)
    K = np.concatenate([k, kt])
    V = np.concatenate([v, vt])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=torch.from_numpy(mask)[None])[0].numpy()
    np.testing.assert_allclose(O_s.reshape(L, d), ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Ohat.reshape(L, d), g[:, None] * ref, rtol=1e-10, atol=1e-12)
    s = (q @ K.T) / math.sqrt(d)
    s[~mask] = -np.inf
    np.testing.assert_allclose(lse.reshape(L), logsumexp(s, axis=1), rtol=1e-12)


def test_text_softmax_off_or_empty_text_is_video_only():
    F, N, d = 20, 3, 8
    q, k, v = (_rand((F, N, d), s) for s in (1, 2, 3))
    kt, vt = _rand((6, d), 4), _rand((6, d), 5)
    base = O.softmax_branch(q, k, v, np.ones((F, N)))
    off = O.softmax_branch(q, k, v, np.ones((F, N)), O.Params(), kt, vt)
    empty = O.softmax_branch(q, k, v, np.ones((F, N)), TEXT, kt[:0], vt[:0])
    for a, b, c in zip(base, off, empty):
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(a, c)


def test_text_softmax_uniform_keys_closed_form():
    # Every key equal: each visible key (video frame tokens once each, every
    # text token) gets the same weight, so the output is the mean of their
    # values.  Video values carry their frame index, text values 100.
    F, N, T, d = 20, 2, 5, 16
    k = np.zeros((F, N, d))
    k[..., 0] = 2.0
    kt = np.zeros((T, d))
    kt[:, 0] = 2.0
    q = np.zeros((F, N, d))
    q[..., 0] = 1.0
    v = np.repeat(np.arange(F, dtype=np.float64)[:, None, None], N, axis=1).repeat(d, axis=2)
    vt = np.full((T, d), 100.0)
    O_s, _, lse = O.softmax_branch(q, k, v, np.ones((F, N)), TEXT, kt, vt)
    for t in range(F):
        fr = [f for f in range(F) if O.visibility(F)[t, f]]
        n_keys = len(fr) * N + T
        want = (N * sum(fr) + 100.0 * T) / n_keys
        np.testing.assert_allclose(O_s[t], want, rtol=1e-13)
        np.testing.assert_allclose(lse[t], 0.5 + math.log(n_keys), rtol=1e-13)


@pytest.mark.parametrize("anchors", [True, False])
def test_text_softmax_is_one_normalisation_split_in_two(anchors):
    # One softmax over (video keys + text keys) equals the two partial
    # softmaxes recombined by their log-sum-exp weights; a separately
    # normalised text attention (the other reading) would not satisfy this.
    F, N, T, d = 15, 3, 7, 8
    p = O.Params(anchors=anchors, text_softmax=True)
    pv = dataclasses.replace(p, text_softmax=False)
    q, k, v = (_rand((F, N, d), s) for s in (11, 12, 13))
    kt, vt = _rand((T, d), 14), _rand((T, d), 15)
    Oj, _, lj = O.softmax_branch(q, k, v, np.ones((F, N)), p, kt, vt)
    Ov, _, lv = O.softmax_branch(q, k, v, np.ones((F, N)), pv)
    st = (q.reshape(-1, d) @ kt.T) / math.sqrt(d)
    lt = logsumexp(st, axis=1).reshape(F, N)
    Ot = (softmax(st, axis=1) @ vt).reshape(F, N, d)
    np.testing.assert_allclose(lj, np.logaddexp(lv, lt), rtol=1e-12)
    wv = np.exp(lv - lj)[..., None]
    wt = np.exp(lt - lj)[..., None]
    np.testing.assert_allclose(Oj, wv * Ov + wt * Ot, rtol=1e-10, atol=1e-12)


def test_text_softmax_dominant_text_key():
    # A text key aligned with every query at a logit 60 above all others
    # takes the whole weight (remaining mass < 2^-80 relative).
    F, N, T, d = 10, 2, 4, 4
    q = np.zeros((F, N, d))
    q[..., 0] = 1.0
    k = _rand((F, N, d), 21) * 0.1
    kt = np.zeros((T, d))
    kt[2, 0] = 120.0          # logit 120 / sqrt(4) = 60
    v = _rand((F, N, d), 22)
    vt = _rand((T, d), 23)
    O_s, _, lse = O.softmax_branch(q, k, v, np.ones((F, N)), TEXT, kt, vt)
    np.testing.assert_allclose(O_s, np.broadcast_to(vt[2], O_s.shape), rtol=1e-12, atol=1e-20)
    np.testing.assert_allclose(lse, 60.0, rtol=1e-12)


def test_text_softmax_leaves_linear_branch_and_rows_consistent():
    F, N, T, d = 10, 3, 4, 8
    rng = np.random.default_rng(31)
    L = F * N
    h = dict(q=rng.standard_normal((L, d)), k=rng.standard_normal((L, d)) * 0.3,
             v=rng.standard_normal((L, d)), beta=rng.random(L), alpha=0.5 + 0.5 * rng.random((F, d)),
             k_text=rng.standard_normal((T, d)) * 0.3, v_text=rng.standard_normal((T, d)),
             beta_text=rng.random(T), g_s=rng.random(L), g_l=rng.random(L))
    r0 = O.vdn_head(**h)
    r1 = O.vdn_head(**h, p=TEXT)
    for key in ("S_text", "P_fwd", "P_rev", "O_l", "Ohat_l"):
        np.testing.assert_array_equal(r0[key], r1[key])
    assert np.abs(r1["O_s"] - r0["O_s"]).max() > 1e-3
    np.testing.assert_allclose(r1["Ohat_s"], h["g_s"][:, None] * r1["O_s"], rtol=1e-13)
    rows = np.array([0, 2, 3, 14, 28, 29])
    rr = O.head_rows(**h, rows=rows, p=TEXT)
    for key in ("O_s", "Ohat_s", "lse"):
        np.testing.assert_allclose(rr[key], r1[key][rows], rtol=1e-12, atol=1e-14)
