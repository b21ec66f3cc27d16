"""Pins of the CPU oracle against what the page and the mathematics fix.

None of these re-type the oracle's own formulas: each compares it with a
hand-written fixture, a closed form, an invariant, a library routine on a
different computational route, or brute force on tiny inputs.  Sources are
the page "Video DeltaNet: A Video-Native Hybrid Attention for Livestream
Video Generation" (papers.paperslantern.ai), cited by section.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import vdn_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden_mask(name):
    rows = [ln.strip() for ln in open(os.path.join(HERE, "golden", name))
            if ln.strip() and not ln.startswith("#")]
    return np.array([[int(c) for c in r] for r in rows], np.uint8)


# ---------------------------------------------------------------------------
# P1: Softmax window + anchor mask (method, local Softmax window)
# ---------------------------------------------------------------------------
def test_mask_matches_hand_written_F20():
    np.testing.assert_array_equal(O.visibility(20), _golden_mask("window_mask_F20.txt"))


@pytest.mark.parametrize("C", range(4, 41))
def test_mask_row_counts_closed_form(C):
    # Counting from the rule: anchor rows see all F frames; non-anchor rows
    # of the edge chunks see 2 chunks + the far anchor (11); rows of chunks
    # 1 and C-2 see 3 chunks, one of which holds an anchor, + the other (16);
    # interior rows see a 15-frame window + both anchors (17).
    F = 5 * C
    m = O.visibility(F)
    rs = m.sum(axis=1)
    assert rs[0] == F and rs[F - 1] == F
    assert all(rs[t] == 11 for t in list(range(1, 5)) + list(range(F - 5, F - 1)))
    assert all(rs[t] == 16 for t in list(range(5, 10)) + list(range(F - 10, F - 5)))
    assert all(rs[t] == 17 for t in range(10, F - 10))
    assert m.sum() == 95 * C - 92
    assert O.visible_pairs(F) == 95 * C - 92


@pytest.mark.parametrize("F", [2, 3, 5, 7, 10])
def test_mask_short_clips_are_dense(F):
    assert O.visibility(F).all()


def test_mask_window_is_15_frames_in_interior():
    # "a 15-frame window except at sequence boundaries"
    F = 60
    for t in range(10, 50):
        lo, hi = O.window_bounds(t, F)
        assert hi - lo + 1 == 15 and lo <= t <= hi


def test_mask_symmetry():
    # the rule is symmetric between query and key frames (four-way anchors,
    # symmetric +-1 chunk window)
    for F in (15, 20, 35, 60):
        m = O.visibility(F)
        np.testing.assert_array_equal(m, m.T)


# ---------------------------------------------------------------------------
# P2: linear regions (method, bidirectional linear attention)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("F", list(range(2, 61)))
def test_regions_partition(F):
    p = O.Params()
    for t in range(F):
        fwd, rev = O.linear_regions(t, F, p)
        vis = O.visible_frames(t, F, p)
        assert not (fwd & rev) and not (fwd & vis) and not (rev & vis)
        assert fwd | rev | vis == set(range(F))
        assert 0 not in fwd | rev and F - 1 not in fwd | rev
        if fwd:
            assert max(fwd) < t
        if rev:
            assert min(rev) > t
        if t in (0, F - 1):
            assert not fwd and not rev and vis == set(range(F))


@pytest.mark.parametrize("F", list(range(2, 61)))
def test_scan_indices_agree_with_regions(F):
    # The gather index and bridge start of the scan form must reproduce the
    # brute-force regions exactly: forward region = non-anchor frames before
    # frame ws; bridge = ws..t; likewise backwards.
    p = O.Params()
    C = -(-F // 5)
    i_f, ws, i_r, we = O.scan_indices(F, p)
    for t in range(F):
        fwd, rev = O.linear_regions(t, F, p)
        assert ws[t] == 5 * i_f[t] and 0 <= i_f[t] <= C and 0 <= i_r[t] <= C
        assert fwd == {f for f in range(0, ws[t]) if f not in (0, F - 1)}
        assert rev == {f for f in range(we[t] + 1, F) if f not in (0, F - 1)}
        assert ws[t] <= t <= we[t]
        if t not in (0, F - 1):
            assert min(i_r[t] * 5, F) - 1 == we[t]


# ---------------------------------------------------------------------------
# Worked scalar example with a closed form (d = 1, N = 1, unit keys,
# constant gates): pins region sizes, the bridge length, the text init
# split, decay-before-write and the (1 + beta) normalisation.
# ---------------------------------------------------------------------------
def _scalar_inputs(F, a, b, v, bt, vt):
    Kf = np.ones((F, 1, 1))
    Vf = np.full((F, 1, 1), v)
    bf = np.full((F, 1), b)
    alpha = np.full((F, 1), a)
    S_text = O.text_state(np.ones((1, 1)), np.full((1, 1), vt), np.array([bt]), 1, 1)
    return Kf, Vf, bf, alpha, S_text


def _geom(S, n, r, u):
    # n steps of S <- r S + u
    return r ** n * S + (u * (1 - r ** n) / (1 - r) if n > 0 else 0.0)


@pytest.mark.parametrize("F", [20, 35, 40])
def test_scalar_closed_form(F):
    a, b, v, bt, vt = 0.93, 0.7, 1.3, 0.4, -2.0
    Kf, Vf, bf, alpha, S_text = _scalar_inputs(F, a, b, v, bt, vt)
    # single text token with unit key: S_text = bt vt / (1 + bt)
    assert S_text[0, 0] == pytest.approx(bt * vt / (1 + bt), rel=1e-14)
    s0 = 0.5 * bt * vt / (1 + bt)
    r, u = a / (1 + b), b * v / (1 + b)
    Mf_b, Mr_b = O.directional_memory_bruteforce(Kf, Vf, bf, alpha, S_text)
    P_f, P_r = O.scan_states(Kf, Vf, bf, alpha, S_text)
    Mf_s, Mr_s = O.directional_memory_scan(P_f, P_r, alpha)
    for t in range(F):
        c = t // 5
        if t in (0, F - 1):
            ef, er = a ** (t + 1) * s0, a ** (F - t) * s0
        else:
            lo = 5 * max(c - 1, 0)
            hi = min(5 * (c + 2), F) - 1
            ef = a ** (t + 1) * s0 if lo == 0 else \
                a ** (t - lo + 1) * _geom(a * s0, lo - 1, r, u)
            er = a ** (F - t) * s0 if hi == F - 1 else \
                a ** (hi - t + 1) * _geom(a * s0, F - 2 - hi, r, u)
        for M_f, M_r in ((Mf_b, Mr_b), (Mf_s, Mr_s)):
            assert M_f[t, 0, 0] == pytest.approx(ef, rel=1e-12, abs=1e-15)
            assert M_r[t, 0, 0] == pytest.approx(er, rel=1e-12, abs=1e-15)


# ---------------------------------------------------------------------------
# P4: the VDA joint frame update (Video Delta Attention section)
# ---------------------------------------------------------------------------
def _rand_frame(rng, N=6, dk=4, dv=3, dup=False):
    K = rng.standard_normal((N, dk))
    if dup:
        K[1] = K[0]
        K[3] = 0.999 * K[2]
    V = rng.standard_normal((N, dv))
    beta = rng.random(N)
    alpha = rng.random(dk)
    S_prev = rng.standard_normal((dk, dv))
    return K, V, beta, alpha, S_prev


def _objective(S, S_tilde, K, V, beta):
    # 1/2 ||S - S~||^2 + 1/2 sum_i beta_i ||k_i^T S - v_i^T||^2, token by token
    J = 0.5 * float(np.sum((S - S_tilde) ** 2))
    for i in range(K.shape[0]):
        r = K[i] @ S - V[i]
        J += 0.5 * beta[i] * float(r @ r)
    return J


@pytest.mark.parametrize("seed", range(5))
def test_vda_update_minimises_the_joint_objective(seed):
    rng = np.random.default_rng(seed)
    K, V, beta, alpha, S_prev = _rand_frame(rng, dup=(seed % 2 == 1))
    S = O.vda_update(S_prev, K, V, beta, alpha)
    S_tilde = alpha[:, None] * S_prev
    J0 = _objective(S, S_tilde, K, V, beta)
    for _ in range(20):
        E = rng.standard_normal(S.shape)
        for eps in (1e-3, 1e-1):
            assert _objective(S + eps * E, S_tilde, K, V, beta) > J0
        # central-difference directional derivative is zero at the minimum
        h = 1e-5
        dJ = (_objective(S + h * E, S_tilde, K, V, beta)
              - _objective(S - h * E, S_tilde, K, V, beta)) / (2 * h)
        assert abs(dJ) < 1e-7


@pytest.mark.parametrize("seed", range(5))
def test_vda_update_residual_at_shared_state(seed):
    # "each residual in the joint solution is evaluated at the shared
    # updated state": S = S~ + K^T B (V - K S)
    rng = np.random.default_rng(100 + seed)
    K, V, beta, alpha, S_prev = _rand_frame(rng, N=9, dk=5, dv=4)
    S = O.vda_update(S_prev, K, V, beta, alpha)
    rhs = alpha[:, None] * S_prev + K.T @ (beta[:, None] * (V - K @ S))
    np.testing.assert_allclose(S, rhs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_vda_update_equals_stacked_least_squares(seed):
    # min ||[I; B^1/2 K] S - [S~; B^1/2 V]||, solved column by column by lstsq
    rng = np.random.default_rng(200 + seed)
    K, V, beta, alpha, S_prev = _rand_frame(rng, N=7, dk=4, dv=3)
    S = O.vda_update(S_prev, K, V, beta, alpha)
    sb = np.sqrt(beta)[:, None]
    Abig = np.vstack([np.eye(4), sb * K])
    Bbig = np.vstack([alpha[:, None] * S_prev, sb * V])
    S_ls = np.linalg.lstsq(Abig, Bbig, rcond=None)[0]
    np.testing.assert_allclose(S, S_ls, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_vda_update_equals_token_space_woodbury(seed):
    # the same update with the inverse taken in token space (N x N)
    rng = np.random.default_rng(300 + seed)
    K, V, beta, alpha, S_prev = _rand_frame(rng, N=5, dk=8, dv=3)
    S = O.vda_update(S_prev, K, V, beta, alpha)
    St = alpha[:, None] * S_prev
    sb = np.sqrt(beta)
    G = np.eye(5) + (sb[:, None] * K) @ (K.T * sb[None, :])
    S_w = St + (K.T * sb[None, :]) @ np.linalg.solve(G, sb[:, None] * (V - K @ St))
    np.testing.assert_allclose(S, S_w, rtol=1e-11, atol=1e-12)


def test_vda_update_affine_map_form():
    rng = np.random.default_rng(7)
    K, V, beta, alpha, S_prev = _rand_frame(rng)
    T, U = O.frame_map(K, V, beta, alpha)
    np.testing.assert_allclose(T @ S_prev + U, O.vda_update(S_prev, K, V, beta, alpha),
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P5: reductions to known rules (Video Delta Attention section)
# ---------------------------------------------------------------------------
def test_single_token_is_the_delta_rule():
    # N = 1, unit key: the classical delta rule with strength beta/(1+beta)
    rng = np.random.default_rng(11)
    dk, dv = 6, 4
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    b = 0.8
    alpha = rng.random(dk)
    S_prev = rng.standard_normal((dk, dv))
    St = alpha[:, None] * S_prev
    bp = b / (1 + b)
    expect = St + bp * np.outer(k, v - k @ St)
    got = O.vda_update(S_prev, k[None], v[None], np.array([b]), alpha)
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("order_seed", range(3))
def test_orthonormal_keys_equal_sequential_token_updates(order_seed):
    # With orthonormal keys the writes do not interfere: the joint update
    # equals token-by-token delta updates (beta' = beta/(1+beta)) in any order.
    rng = np.random.default_rng(21)
    dk, dv, N = 8, 3, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:N]
    V = rng.standard_normal((N, dv))
    beta = rng.random(N)
    alpha = rng.random(dk)
    S_prev = rng.standard_normal((dk, dv))
    S = alpha[:, None] * S_prev
    for i in np.random.default_rng(order_seed).permutation(N):
        bp = beta[i] / (1 + beta[i])
        S = S + bp * np.outer(K[i], V[i] - K[i] @ S)
    np.testing.assert_allclose(O.vda_update(S_prev, K, V, beta, alpha), S,
                               rtol=1e-12, atol=1e-12)


def test_small_beta_limit_is_the_frozen_state_update():
    # Eq. (3c): the frozen-state batched update S~ + K^T B (V - K S~).  VDA
    # differs from it by O(beta^2).
    rng = np.random.default_rng(31)
    K, V, beta0, alpha, S_prev = _rand_frame(rng, N=12, dk=5, dv=3)
    St = alpha[:, None] * S_prev
    errs = []
    for s in (1e-2, 5e-3, 2.5e-3):
        beta = s * beta0
        frozen = St + K.T @ (beta[:, None] * (V - K @ St))
        errs.append(np.linalg.norm(O.vda_update(S_prev, K, V, beta, alpha) - frozen))
    assert 3.6 < errs[0] / errs[1] < 4.4 and 3.6 < errs[1] / errs[2] < 4.4


# ---------------------------------------------------------------------------
# P6: Proposition 1, non-expansive inherited-state transition
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(10))
def test_prop1_transition_is_non_expansive(seed):
    rng = np.random.default_rng(400 + seed)
    K, V, beta, alpha, _ = _rand_frame(rng, N=40, dk=6, dv=3, dup=True)
    beta = beta * 5.0            # any beta >= 0
    T, _U = O.frame_map(K, V, beta, alpha)
    assert np.linalg.svd(T, compute_uv=False)[0] <= 1 + 1e-12
    D = rng.standard_normal((6, 3))
    assert np.linalg.norm(T @ D) <= np.linalg.norm(D) * (1 + 1e-12)


def test_frozen_state_transition_can_expand():
    # the contrast the page draws: without frame-size key scaling the
    # additive frozen-state transition (I - A) diag(alpha) can amplify
    rng = np.random.default_rng(5)
    K = rng.standard_normal((64, 4))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    A, _ = O.frame_stats(K, np.zeros((64, 1)), np.full(64, 0.9))
    assert np.linalg.svd(np.eye(4) - A, compute_uv=False)[0] > 1


# ---------------------------------------------------------------------------
# P7: gate invariants and the text state
# ---------------------------------------------------------------------------
def _rand_head(rng, F=20, N=3, dk=4, dv=3, T=5):
    L = F * N
    return dict(q=rng.standard_normal((L, dk)), k=rng.standard_normal((L, dk)),
                v=rng.standard_normal((L, dv)), beta=rng.random(L),
                alpha=0.8 + 0.2 * rng.random((F, dk)),
                k_text=rng.standard_normal((T, dk)), v_text=rng.standard_normal((T, dv)),
                beta_text=rng.random(T), g_s=rng.random(L), g_l=rng.random(L))


def test_zero_beta_unit_alpha_counts_the_prompt_once():
    rng = np.random.default_rng(41)
    h = _rand_head(rng)
    h["beta"][:] = 0
    h["alpha"][:] = 1
    r = O.vdn_head(**h, want_softmax=False)
    S_text = r["S_text"]
    for t in range(20):
        np.testing.assert_allclose(r["M_fwd"][t], 0.5 * S_text, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r["M_rev"][t], 0.5 * S_text, rtol=1e-13, atol=1e-14)
    # readout q^T S_text, token by token with explicit sums
    q = h["q"]
    for l in (0, 7, 31, 59):
        expect = [sum(q[l, i] * S_text[i, j] for i in range(4)) for j in range(3)]
        np.testing.assert_allclose(r["O_l"][l], expect, rtol=1e-12, atol=1e-14)


def test_zero_beta_memory_is_decayed_text_state():
    rng = np.random.default_rng(42)
    F = 25
    h = _rand_head(rng, F=F)
    h["beta"][:] = 0
    r = O.vdn_head(**h, want_softmax=False)
    a = h["alpha"]
    for t in range(F):
        df = np.prod(a[:t + 1], axis=0)
        dr = np.prod(a[t:], axis=0)
        np.testing.assert_allclose(r["M_fwd"][t], df[:, None] * 0.5 * r["S_text"], rtol=1e-12)
        np.testing.assert_allclose(r["M_rev"][t], dr[:, None] * 0.5 * r["S_text"], rtol=1e-12)


def test_no_text_tokens_zero_state():
    assert not O.text_state(np.zeros((0, 4)), np.zeros((0, 3)), np.zeros(0), 4, 3).any()


def test_text_state_is_one_update_from_zero():
    rng = np.random.default_rng(43)
    Kt, Vt, bt = rng.standard_normal((6, 4)), rng.standard_normal((6, 3)), rng.random(6)
    S = O.text_state(Kt, Vt, bt, 4, 3)
    # minimiser of 1/2||S||^2 + 1/2 sum b||k^T S - v||^2: normal equation by lstsq
    sb = np.sqrt(bt)[:, None]
    S_ls = np.linalg.lstsq(np.vstack([np.eye(4), sb * Kt]),
                           np.vstack([np.zeros((4, 3)), sb * Vt]), rcond=None)[0]
    np.testing.assert_allclose(S, S_ls, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# P8: brute-force masked recurrences == chunk-boundary scan + gather/bridge
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("F,params", [
    (20, O.Params()), (25, O.Params()), (40, O.Params()), (23, O.Params()),
    (18, O.Params(chunk_frames=3, window_chunks=2)),
    (20, O.Params(anchors=False)), (12, O.Params(chunk_frames=4, window_chunks=0)),
    (2, O.Params()), (5, O.Params()), (10, O.Params()),
])
def test_bruteforce_equals_scan(F, params):
    rng = np.random.default_rng(F)
    h = _rand_head(rng, F=F)
    rb = O.vdn_head(**h, p=params, linear_form="bruteforce", want_softmax=False)
    rs = O.vdn_head(**h, p=params, linear_form="scan", want_softmax=False)
    np.testing.assert_allclose(rs["M_fwd"], rb["M_fwd"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(rs["M_rev"], rb["M_rev"], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(rs["O_l"], rb["O_l"], rtol=1e-10, atol=1e-12)


def test_scan_states_at_chunk_boundaries_match_direct_recurrence():
    # P_fwd[i] is the state after exactly i chunks: run the VDA updates
    # directly (no affine maps) and compare at every boundary.
    rng = np.random.default_rng(51)
    F, N, dk, dv = 20, 3, 4, 3
    h = _rand_head(rng, F=F, N=N)
    Kf = h["k"].reshape(F, N, dk)
    Vf = h["v"].reshape(F, N, dv)
    bf = h["beta"].reshape(F, N)
    S_text = O.text_state(h["k_text"], h["v_text"], h["beta_text"], dk, dv)
    P_f, P_r = O.scan_states(Kf, Vf, bf, h["alpha"], S_text)
    S = 0.5 * S_text
    for f in range(F):
        if f in (0, F - 1):
            S = h["alpha"][f][:, None] * S
        else:
            S = O.vda_update(S, Kf[f], Vf[f], bf[f], h["alpha"][f])
        if (f + 1) % 5 == 0:
            np.testing.assert_allclose(P_f[(f + 1) // 5], S, rtol=1e-12, atol=1e-13)
    S = 0.5 * S_text
    for f in range(F - 1, -1, -1):
        if f in (0, F - 1):
            S = h["alpha"][f][:, None] * S
        else:
            S = O.vda_update(S, Kf[f], Vf[f], bf[f], h["alpha"][f])
        if f % 5 == 0:
            np.testing.assert_allclose(P_r[f // 5], S, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# P3: windowed Softmax == dense masked Softmax (torch SDPA, fp64)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("F,N,d", [(20, 4, 8), (35, 3, 16), (7, 5, 4)])
def test_softmax_equals_dense_masked_sdpa(F, N, d):
    rng = np.random.default_rng(F * 100 + N)
    L = F * N
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    g = rng.random(L)
    O_s, Ohat, lse = O.softmax_branch(q.reshape(F, N, d), k.reshape(F, N, d),
                                      v.reshape(F, N, d), g.reshape(F, N))
    fm = O.visibility(F).astype(bool)
    tok = np.repeat(np.repeat(fm, N, axis=0), N, axis=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(tok)[None])[0].numpy()
    np.testing.assert_allclose(O_s.reshape(L, d), ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(Ohat.reshape(L, d), g[:, None] * ref, rtol=1e-10, atol=1e-12)
    # lse against a log-sum-exp over the dense masked logits (scipy route)
    from scipy.special import logsumexp
    s = (q @ k.T) / math.sqrt(d)
    s[~tok] = -np.inf
    np.testing.assert_allclose(lse.reshape(L), logsumexp(s, axis=1), rtol=1e-12)


def test_softmax_uniform_keys_average_each_visible_frame_once():
    # Equal keys give uniform attention: the output is the mean of the
    # visible values, so double counting an anchor would show.  Values carry
    # their frame index; q.k = 2 and dk = 16 give logit 0.5 (scale 1/sqrt dk).
    F, N, d = 20, 2, 16
    k = np.zeros((F, N, d))
    k[..., 0] = 2.0
    q = np.zeros((F, N, d))
    q[..., 0] = 1.0
    v = np.repeat(np.arange(F, dtype=np.float64)[:, None, None], N, axis=1).repeat(d, axis=2)
    O_s, _, lse = O.softmax_branch(q, k, v, np.ones((F, N)))
    expect_sets = {0: range(20), 19: range(20)}
    for t in range(1, 5):
        expect_sets[t] = list(range(10)) + [19]
    for t in range(5, 10):
        expect_sets[t] = list(range(15)) + [19]
    for t in range(10, 15):
        expect_sets[t] = [0] + list(range(5, 20))
    for t in range(15, 19):
        expect_sets[t] = [0] + list(range(10, 20))
    for t, fr in expect_sets.items():
        fr = list(fr)
        np.testing.assert_allclose(O_s[t], np.mean(fr), rtol=1e-13)
        np.testing.assert_allclose(lse[t], 0.5 + math.log(len(fr) * N), rtol=1e-13)


# ---------------------------------------------------------------------------
# P10: epilogue and merge (method, branch calibration)
# ---------------------------------------------------------------------------
def test_rms_norm_rows_have_unit_rms_per_token_and_head():
    rng = np.random.default_rng(61)
    x = rng.standard_normal((7, 5, 16)) * rng.random((7, 5, 1)) * 10
    y = O.rms_norm(x, None, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-9)
    # per-row scaling invariance (the normalised axis is the last one only)
    y2 = O.rms_norm(x * rng.random((7, 5, 1)), None, 0.0)
    np.testing.assert_allclose(y, y2, rtol=1e-9)


def test_linear_gate_zero_and_one():
    rng = np.random.default_rng(62)
    h = _rand_head(rng)
    h["g_l"][:] = 0
    assert not O.vdn_head(**h, want_softmax=False)["Ohat_l"].any()
    h["g_l"][:] = 1
    r = O.vdn_head(**h, want_softmax=False)
    np.testing.assert_allclose(np.sqrt(np.mean(r["Ohat_l"] ** 2, axis=-1)),
                               np.sqrt(np.mean(r["O_l"] ** 2, axis=-1)
                                       / (np.mean(r["O_l"] ** 2, axis=-1) + 1e-6)),
                               rtol=1e-12)


def test_merge_projection_layout():
    rng = np.random.default_rng(63)
    B, L, H, dv, D = 2, 5, 3, 4, 7
    Os = rng.standard_normal((B, L, H, dv))
    Ol = rng.standard_normal((B, L, H, dv))
    Ws = rng.standard_normal((H * dv, D))
    Wl = rng.standard_normal((H * dv, D))
    out = O.merge(Os, Ol, Ws, Wl)
    # element by element: out[b,l,:] = sum_h sum_j Os[b,l,h,j] Ws[h*dv+j,:] + ...
    for b in range(B):
        for l in range(L):
            e = np.zeros(D)
            for hh in range(H):
                for j in range(dv):
                    e += Os[b, l, hh, j] * Ws[hh * dv + j] + Ol[b, l, hh, j] * Wl[hh * dv + j]
            np.testing.assert_allclose(out[b, l], e, rtol=1e-12, atol=1e-12)
    # a block-identity W_s selects one head; zero W_l drops the linear branch
    Ws1 = np.zeros((H * dv, dv))
    Ws1[1 * dv:2 * dv] = np.eye(dv)
    np.testing.assert_allclose(O.merge(Os, Ol, Ws1, np.zeros((H * dv, dv))), Os[:, :, 1])
    np.testing.assert_allclose(O.merge(Os, Ol), Os + Ol)


def test_full_operator_small_case_consistent():
    # both linear forms through the whole operator agree; the output is the
    # merge of the per-head gated branches
    from vdn_inputs import CONFIGS, full_inputs
    cfg = CONFIGS["tiny"].replace(F=10, N=4, H=2)
    inp = full_inputs(cfg)
    r1 = O.vdn_attn(inp, linear_form="scan")
    r2 = O.vdn_attn(inp, linear_form="bruteforce")
    np.testing.assert_allclose(r1["out"], r2["out"], rtol=1e-11, atol=1e-12)
    assert r1["out"].shape == (1, cfg.L, cfg.D)


# ---------------------------------------------------------------------------
# head_rows: the sampled-row evaluator behind the full-size GPU checks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("p", [
    O.Params(),
    O.Params(chunk_frames=3, window_chunks=2, text_softmax=True, text_init_scale=0.8,
             rms_eps=1e-3, softmax_scale=0.3),
    O.Params(anchors=False, chunk_frames=4, window_chunks=0, text_softmax=True),
])
def test_head_rows_matches_full_head(p):
    """head_rows at shuffled rows equals the full per-head evaluation: the
    linear leg against each query frame's own masked recurrence
    (vdn_head's brute-force form), the Softmax leg against torch's dense
    softmax with the visibility mask and the text columns.  Gates g_s and
    g_l differ, so using one for the other fails."""
    rng = np.random.default_rng(11)
    F, N, d, T = 24, 3, 4, 5
    L = F * N
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q = rng.standard_normal((L, d))
    k = unit(rng.standard_normal((L, d)))
    v = rng.standard_normal((L, d))
    beta = rng.random(L)
    alpha = rng.uniform(0.7, 1.0, (F, d))
    kt, vt, bt = unit(rng.standard_normal((T, d))), rng.standard_normal((T, d)), rng.random(T)
    g_s, g_l = rng.random(L), rng.random(L)
    gamma = rng.uniform(0.5, 1.5, d)
    rows = rng.permutation(L)[: L // 2]
    got = O.head_rows(q, k, v, beta, alpha, kt, vt, bt, g_s, g_l, rows, gamma=gamma, p=p)
    ref = O.vdn_head(q, k, v, beta, alpha, kt, vt, bt, g_s, g_l, gamma=gamma, p=p, F=F,
                     linear_form="bruteforce", want_softmax=False)
    np.testing.assert_allclose(got["O_l"], ref["O_l"][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["Ohat_l"], ref["Ohat_l"][rows], rtol=1e-10, atol=1e-12)
    # Softmax leg: dense masked softmax in torch (fp64)
    scale = 1 / math.sqrt(d) if p.softmax_scale is None else p.softmax_scale
    frame_mask = torch.from_numpy(O.visibility(F, p).astype(bool))
    mask = frame_mask.repeat_interleave(N, 0).repeat_interleave(N, 1)       # [L, L]
    Kall, Vall = torch.from_numpy(k), torch.from_numpy(v)
    if p.text_softmax:
        Kall = torch.cat([Kall, torch.from_numpy(kt)])
        Vall = torch.cat([Vall, torch.from_numpy(vt)])
        mask = torch.cat([mask, torch.ones(L, T, dtype=torch.bool)], dim=1)
    logits = (torch.from_numpy(q) @ Kall.T) * scale
    logits = logits.masked_fill(~mask, float("-inf"))
    O_s = torch.softmax(logits, dim=1) @ Vall
    lse = torch.logsumexp(logits, dim=1)
    np.testing.assert_allclose(got["O_s"], O_s.numpy()[rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["Ohat_s"], g_s[rows, None] * O_s.numpy()[rows], rtol=1e-10,
                               atol=1e-12)
    np.testing.assert_allclose(got["lse"], lse.numpy()[rows], rtol=1e-12)
    # the states are the full-head ones
    full = O.vdn_head(q, k, v, beta, alpha, kt, vt, bt, g_s, g_l, gamma=gamma, p=p, F=F,
                      want_softmax=False)
    for key in ("P_fwd", "P_rev", "S_text"):
        np.testing.assert_allclose(got[key], full[key], rtol=1e-12, atol=1e-14)
