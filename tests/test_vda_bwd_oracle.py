"""Pins of the linear-branch (VDA) backward oracle.

- torch autograd (fp64) through an independent torch forward written in the
  brute-force form: every query frame runs its own masked frame recurrence
  with torch.linalg.solve -- no chunk states, no gather/bridge, no frame
  maps -- so it shares no arithmetic with the oracle's adjoint;
- central finite differences on the forward oracle itself;
- identities every correct gradient obeys: with eps = 0 RMSNorm is scale
  invariant, so q . dq = 0 on every token; sum_j gamma_j dgamma_j equals
  sum_tokens g_l dg_l; a zero write gate blocks every gradient into the video
  keys and values.
"""
import numpy as np
import pytest
import torch

from oracle import vda_bwd as VB
from oracle import vdn_oracle as O

KEYS = ("q", "k", "v", "beta", "alpha", "k_text", "v_text", "beta_text", "g_l", "gamma")


def _case(F, N, d, T, seed, alpha_lo=0.5):
    rng = np.random.default_rng(seed)
    L = F * N
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    return dict(q=rng.standard_normal((L, d)), k=unit(rng.standard_normal((L, d))),
                v=rng.standard_normal((L, d)), beta=rng.random(L) * 2,
                alpha=rng.uniform(alpha_lo, 1.0, (F, d)), k_text=unit(rng.standard_normal((T, d))),
                v_text=rng.standard_normal((T, d)), beta_text=rng.random(T) * 2,
                g_l=rng.random(L), gamma=rng.uniform(0.5, 1.5, d)), rng.standard_normal((L, d))


def _oracle_grads(x, dO, p):
    return VB.linear_branch_bwd(x["q"], x["k"], x["v"], x["beta"], x["alpha"], x["k_text"],
                                x["v_text"], x["beta_text"], x["g_l"], x["gamma"], dO, p)


def _torch_head_ohat(t_, F, p):
    """Ohat_l [L, d] of one head in torch, in the brute-force form (method,
    bidirectional linear attention: each query frame's own forward and
    reverse masked recurrence).  t_: torch tensors of one head's inputs."""
    L, d = t_["q"].shape
    N = L // F
    eye = torch.eye(d, dtype=torch.float64)

    def update(S, K, V, b, al):
        A = K.T @ (b[:, None] * K)
        W = K.T @ (b[:, None] * V)
        return torch.linalg.solve(eye + A, al[:, None] * S + W)

    S_text = update(torch.zeros(d, d, dtype=torch.float64), t_["k_text"], t_["v_text"],
                    t_["beta_text"], torch.ones(d, dtype=torch.float64))
    S0 = p.text_init_scale * S_text
    outs = []
    for t in range(F):
        fwd, rev = O.linear_regions(t, F, p)
        rows = slice(t * N, (t + 1) * N)
        mems = []
        for region, order in ((fwd, range(0, t + 1)), (rev, range(F - 1, t - 1, -1))):
            S = S0
            for f in order:
                fr = slice(f * N, (f + 1) * N)
                if f in region:
                    S = update(S, t_["k"][fr], t_["v"][fr], t_["beta"][fr], t_["alpha"][f])
                else:
                    S = t_["alpha"][f][:, None] * S
            mems.append(S)
        Ot = t_["q"][rows] @ (mems[0] + mems[1])
        r = torch.sqrt(torch.mean(Ot * Ot, dim=1, keepdim=True) + p.rms_eps)
        outs.append(t_["g_l"][rows][:, None] * t_["gamma"] * Ot / r)
    return torch.cat(outs)


def _torch_grads(x, dO, p):
    """Autograd through the brute-force forward (method, bidirectional linear
    attention: each query frame's own forward and reverse masked recurrence)."""
    F = x["alpha"].shape[0]
    t_ = {kk: torch.tensor(x[kk], dtype=torch.float64, requires_grad=True) for kk in KEYS}
    L, d = x["q"].shape
    N = L // F
    eye = torch.eye(d, dtype=torch.float64)

    def update(S, K, V, b, al):
        A = K.T @ (b[:, None] * K)
        W = K.T @ (b[:, None] * V)
        return torch.linalg.solve(eye + A, al[:, None] * S + W)

    S_text = update(torch.zeros(d, d, dtype=torch.float64), t_["k_text"], t_["v_text"],
                    t_["beta_text"], torch.ones(d, dtype=torch.float64))
    S0 = p.text_init_scale * S_text
    loss = 0
    for t in range(F):
        fwd, rev = O.linear_regions(t, F, p)
        rows = slice(t * N, (t + 1) * N)
        mems = []
        for region, order in ((fwd, range(0, t + 1)), (rev, range(F - 1, t - 1, -1))):
            S = S0
            for f in order:
                fr = slice(f * N, (f + 1) * N)
                if f in region:
                    S = update(S, t_["k"][fr], t_["v"][fr], t_["beta"][fr], t_["alpha"][f])
                else:
                    S = t_["alpha"][f][:, None] * S
            mems.append(S)
        Ot = t_["q"][rows] @ (mems[0] + mems[1])
        r = torch.sqrt(torch.mean(Ot * Ot, dim=1, keepdim=True) + p.rms_eps)
        Oh = t_["g_l"][rows][:, None] * t_["gamma"] * Ot / r
        loss = loss + torch.sum(Oh * torch.from_numpy(dO[rows]))
    loss.backward()
    return {kk: t_[kk].grad.numpy() for kk in KEYS}


@pytest.mark.parametrize("F,N,d,T,anchors,cf,wc", [
    (20, 3, 4, 3, True, 5, 1),       # four chunks: every region kind
    (30, 2, 4, 2, True, 5, 1),       # six chunks: interior chunks with both regions
    (12, 2, 3, 2, False, 3, 1),      # no anchors, 3-frame chunks
    (18, 2, 4, 3, True, 3, 2),       # wider window
    (17, 2, 3, 2, True, 5, 1),       # partial last chunk (oracle-only case)
])
def test_matches_torch_autograd_bruteforce(F, N, d, T, anchors, cf, wc):
    p = O.Params(anchors=anchors, chunk_frames=cf, window_chunks=wc)
    x, dO = _case(F, N, d, T, seed=F * 100 + N * 10 + d)
    got = _oracle_grads(x, dO, p)
    want = _torch_grads(x, dO, p)
    for key in KEYS:
        g = got["d" + key]
        assert g.shape == want[key].shape, key
        np.testing.assert_allclose(g, want[key], rtol=1e-9, atol=1e-11, err_msg=key)


def test_central_finite_differences():
    F, N, d, T = 15, 2, 3, 2
    p = O.Params()
    x, dO = _case(F, N, d, T, seed=7)

    def loss(xx):
        r = O.vdn_head(xx["q"], xx["k"], xx["v"], xx["beta"], xx["alpha"], xx["k_text"],
                       xx["v_text"], xx["beta_text"], np.ones(F * N), xx["g_l"], xx["gamma"], p, F,
                       want_softmax=False)
        return float(np.sum(r["Ohat_l"] * dO))

    got = _oracle_grads(x, dO, p)
    rng = np.random.default_rng(1)
    h = 1e-6
    for key in KEYS:
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in x[key].shape)
            xp = {kk: vv.copy() for kk, vv in x.items()}
            xm = {kk: vv.copy() for kk, vv in x.items()}
            xp[key][idx] += h
            xm[key][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            g = got["d" + key][idx]
            assert abs(fd - g) <= 1e-6 * max(1.0, abs(fd)), (key, idx, fd, g)


def test_scale_invariance_without_eps():
    # eps = 0: Ohat is invariant to scaling O_t, so dO is orthogonal to O and q . dq = o . dO = 0
    p = O.Params(rms_eps=0.0)
    x, dO = _case(20, 3, 4, 3, seed=3)
    g = _oracle_grads(x, dO, p)
    qdq = np.sum(x["q"] * g["dq"], axis=1)
    assert np.abs(qdq).max() < 1e-10 * np.abs(g["dq"]).max() * np.abs(x["q"]).max()


def test_gamma_and_gate_gradients_agree():
    p = O.Params()
    x, dO = _case(20, 3, 4, 3, seed=4)
    g = _oracle_grads(x, dO, p)
    np.testing.assert_allclose(np.sum(x["gamma"] * g["dgamma"]), np.sum(x["g_l"] * g["dg_l"]),
                               rtol=1e-12)


def test_zero_write_gate_blocks_video_key_value_gradients():
    p = O.Params()
    x, dO = _case(20, 3, 4, 3, seed=5)
    x["beta"][:] = 0.0
    g = _oracle_grads(x, dO, p)
    assert not g["dk"].any() and not g["dv"].any()
    assert np.abs(g["dbeta"]).max() > 0 and np.abs(g["dk_text"]).max() > 0


def test_stacked_wrapper_matches_autograd_over_all_heads():
    """vda_bwd over [B, H] stacked inputs with a [B, L, H, d] output gradient
    against torch autograd through a stacked forward: every head's Ohat_l in
    the brute-force form, laid out [B, L, H, d] like the operator's output,
    with one gamma shared by all heads (its gradient sums over heads).  The
    gradient is asymmetric in b, h and l, so slicing dOhat on the wrong axis
    or overwriting dgamma per head fails."""
    B, H, F, N, d, T = 2, 3, 20, 2, 3, 2        # four chunks: both regions non-empty
    p = O.Params()
    rng = np.random.default_rng(21)
    L = F * N
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    inp = dict(q=rng.standard_normal((B, H, L, d)), k=unit(rng.standard_normal((B, H, L, d))),
               v=rng.standard_normal((B, H, L, d)), beta=rng.random((B, H, L)),
               alpha=rng.uniform(0.6, 1.0, (B, H, F, d)),
               k_text=unit(rng.standard_normal((B, H, T, d))), v_text=rng.standard_normal((B, H, T, d)),
               beta_text=rng.random((B, H, T)), g_s=rng.random((B, H, L)), g_l=rng.random((B, H, L)),
               gamma=rng.uniform(0.5, 1.5, d))
    dOhat = rng.standard_normal((B, L, H, d))
    got = VB.vda_bwd(inp, dOhat, p)
    per_head = [k for k in KEYS if k != "gamma"]
    leaves = {k: torch.tensor(inp[k], dtype=torch.float64, requires_grad=True) for k in per_head}
    gamma = torch.tensor(inp["gamma"], dtype=torch.float64, requires_grad=True)
    rows = []
    for b in range(B):
        heads = []
        for h in range(H):
            t_ = {k: leaves[k][b, h] for k in per_head}
            t_["gamma"] = gamma
            heads.append(_torch_head_ohat(t_, F, p))          # [L, d]
        rows.append(torch.stack(heads, dim=1))                 # [L, H, d]
    Ohat = torch.stack(rows)                                   # [B, L, H, d]
    torch.sum(Ohat * torch.from_numpy(dOhat)).backward()
    for k in per_head:
        np.testing.assert_allclose(got["d" + k], leaves[k].grad.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg=k)
    np.testing.assert_allclose(got["dgamma"], gamma.grad.numpy(), rtol=1e-9, atol=1e-11)
    # a subset of heads leaves the others at zero
    sub = VB.vda_bwd(inp, dOhat, p, heads=[(1, 2)])
    np.testing.assert_allclose(sub["dq"][1, 2], got["dq"][1, 2], rtol=1e-12)
    assert not sub["dq"][0].any() and not sub["dq"][1, :2].any()
