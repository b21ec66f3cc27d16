"""Backward pass of the linear (VDA) branch -- CPU fp64 oracle.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and shares no code with it.

Source: "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation" (arXiv 2609.20744).  The forward is defined in the Video Delta
Attention section (frame statistics, the joint frame update and its closed
form), the method's bidirectional linear attention (text-initialised scans,
gather + decay bridge, sum of the two readouts) and branch calibration
(RMSNorm + output gate).  The experiments train the model through this
operator (staged adaptation), which needs its gradients; the page prints
none, so they are the chain rule applied to those definitions, step by step
in reverse order, through the page's own quantities:

  epilogue   Ohat = g * gamma * O / r,  r = sqrt(mean(O^2) + eps)
  readout    O_t = Q_t M_t
  bridge     M_t = diag(D_fwd[t]) P_fwd[i_fwd[t]] + diag(D_rev[t]) P_rev[i_rev[t]],
             D_fwd[t] = prod_{f=ws..t} alpha_f,  D_rev[t] = prod_{f=t..we} alpha_f
  states     S_f = T_f S_{f-1} + U_f (forward), S_f = T_f S_{f+1} + U_f (reverse),
             from text_init_scale * S_text; P_* are the states at chunk boundaries
  frame map  T_f = X_f diag(alpha_f), U_f = X_f W_f, X_f = (I + A_f)^{-1}
             (anchor frames: T_f = diag(alpha_f), U_f = 0)
  text       S_text = X_T W_T
  statistics A = K^T diag(beta) K,  W = K^T diag(beta) V

The states are run frame by frame (no chunk composition) and every adjoint
uses the plain matrix identities d(X) = -X d(I + A) X, d(XY) = dX Y + X dY.
Everything in float64.
"""
from __future__ import annotations

import numpy as np

from oracle import vdn_oracle as O


def _frame_states(T, U, S0, order):
    """States along one scan direction: returns {f: state after frame f} and
    the state before the first frame under key None."""
    states = {None: S0}
    S = S0
    for f in order:
        S = T[f] @ S + U[f]
        states[f] = S
    return states


def _excl_prod(a, lo, hi, f):
    """prod_{g = lo..hi, g != f} a[g] (channel-wise), with no division."""
    out = np.ones(a.shape[1])
    for g in range(lo, hi + 1):
        if g != f:
            out = out * a[g]
    return out


def linear_branch_bwd(q, k, v, beta, alpha, k_text, v_text, beta_text, g_l, gamma, dOhat,
                      p: O.Params = O.DEFAULT):
    """Gradients of Ohat_l (one head) with respect to every input of the
    linear branch.

    q, k, v: [L, d] frame-major; beta, g_l: [L]; alpha: [F, dk];
    k_text, v_text: [T, d]; beta_text: [T]; gamma: [dv] or None (= 1);
    dOhat: [L, dv], the gradient of Ohat_l.
    Returns a dict: dq, dk, dv [L, d]; dbeta, dg_l [L]; dalpha [F, dk];
    dk_text, dv_text [T, d]; dbeta_text [T]; dgamma [dv].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.asarray(alpha, np.float64)
    F, dk = a.shape
    L = q.shape[0]
    dv = v.shape[1]
    N = L // F
    cf = p.chunk_frames
    C = -(-F // cf)
    s0 = p.text_init_scale
    Qf, Kf, Vf = q.reshape(F, N, dk), k.reshape(F, N, dk), v.reshape(F, N, dv)
    bf = np.asarray(beta, np.float64).reshape(F, N)
    gl = np.asarray(g_l, np.float64).reshape(F, N)
    gm = np.ones(dv) if gamma is None else np.asarray(gamma, np.float64)
    dOh = np.asarray(dOhat, np.float64).reshape(F, N, dv)
    eye = np.eye(dk)

    # ---- forward, keeping every intermediate ----
    X = np.zeros((F, dk, dk))
    Wst = np.zeros((F, dk, dv))
    T = np.zeros((F, dk, dk))
    U = np.zeros((F, dk, dv))
    for f in range(F):
        if O.is_anchor(f, F, p):
            T[f] = np.diag(a[f])
            continue
        A, Wst[f] = O.frame_stats(Kf[f], Vf[f], bf[f])
        X[f] = np.linalg.inv(eye + A)
        T[f] = X[f] @ np.diag(a[f])
        U[f] = X[f] @ Wst[f]
    has_text = k_text is not None and len(k_text) > 0
    if has_text:
        kt = np.asarray(k_text, np.float64)
        vt = np.asarray(v_text, np.float64)
        bt = np.asarray(beta_text, np.float64)
        A_T, W_T = O.frame_stats(kt, vt, bt)
        X_T = np.linalg.inv(eye + A_T)
        S_text = X_T @ W_T
    else:
        S_text = np.zeros((dk, dv))
    S0 = s0 * S_text
    fwd = _frame_states(T, U, S0, range(F))
    rev = _frame_states(T, U, S0, range(F - 1, -1, -1))
    P_fwd = [S0] + [fwd[min((i + 1) * cf, F) - 1] for i in range(C)]   # P_fwd[i], i = 0..C
    P_rev = [rev[i * cf] for i in range(C)] + [S0]                     # P_rev[i], i = 0..C
    i_fwd, ws, i_rev, we = O.scan_indices(F, p)

    # ---- epilogue and readout, per query frame ----
    dq = np.zeros((F, N, dk))
    dg = np.zeros((F, N))
    dgamma = np.zeros(dv)
    dP_fwd = [np.zeros((dk, dv)) for _ in range(C + 1)]
    dP_rev = [np.zeros((dk, dv)) for _ in range(C + 1)]
    dalpha = np.zeros((F, dk))
    for t in range(F):
        D_f = np.prod(a[ws[t]:t + 1], axis=0)
        D_r = np.prod(a[t:we[t] + 1], axis=0)
        M = D_f[:, None] * P_fwd[i_fwd[t]] + D_r[:, None] * P_rev[i_rev[t]]
        Ot = Qf[t] @ M                                        # [N, dv]
        r = np.sqrt(np.mean(Ot * Ot, axis=1, keepdims=True) + p.rms_eps)
        dg[t] = np.sum(dOh[t] * gm * Ot / r, axis=1)
        dgamma += np.sum(dOh[t] * gl[t][:, None] * Ot / r, axis=0)
        u = gl[t][:, None] * gm * dOh[t]                      # gradient of O / r
        dO = u / r - Ot * np.sum(u * Ot, axis=1, keepdims=True) / (dv * r ** 3)
        dq[t] = dO @ M.T
        dM = Qf[t].T @ dO                                     # [dk, dv]
        dP_fwd[i_fwd[t]] += D_f[:, None] * dM
        dP_rev[i_rev[t]] += D_r[:, None] * dM
        dD_f = np.sum(dM * P_fwd[i_fwd[t]], axis=1)
        dD_r = np.sum(dM * P_rev[i_rev[t]], axis=1)
        for f in range(ws[t], t + 1):
            dalpha[f] += dD_f * _excl_prod(a, ws[t], t, f)
        for f in range(t, we[t] + 1):
            dalpha[f] += dD_r * _excl_prod(a, t, we[t], f)

    # ---- the two frame recurrences, adjoint (reverse order of each scan) ----
    dT = np.zeros_like(T)
    dU = np.zeros_like(U)
    dS_text = np.zeros((dk, dv))
    lam = dP_fwd[C].copy()                                   # adjoint of the last forward state
    for f in range(F - 1, -1, -1):
        prev = fwd[f - 1] if f > 0 else S0
        dT[f] += lam @ prev.T
        dU[f] += lam
        lam = T[f].T @ lam
        if f % cf == 0:                                      # state before frame f is P_fwd[f / cf]
            lam = lam + dP_fwd[f // cf]
    dS_text += s0 * lam
    lam = dP_rev[0].copy()                                   # adjoint of the last reverse state
    for f in range(F):
        prev = rev[f + 1] if f + 1 < F else S0
        dT[f] += lam @ prev.T
        dU[f] += lam
        lam = T[f].T @ lam
        if (f + 1) % cf == 0 or f + 1 == F:                  # state before frame f is P_rev[(f+1)/cf]
            lam = lam + dP_rev[-(-(f + 1) // cf)]
    dS_text += s0 * lam

    # ---- frame maps -> statistics -> tokens ----
    dk_ = np.zeros((F, N, dk))
    dv_ = np.zeros((F, N, dv))
    dbeta = np.zeros((F, N))
    for f in range(F):
        if O.is_anchor(f, F, p):
            dalpha[f] += np.diag(dT[f])                      # T = diag(alpha)
            continue
        dalpha[f] += np.sum(X[f] * dT[f], axis=0)            # T = X diag(alpha)
        dX = dT[f] @ np.diag(a[f]) + dU[f] @ Wst[f].T
        dW = X[f].T @ dU[f]
        dA = -X[f].T @ dX @ X[f].T
        dk_[f], dv_[f], dbeta[f] = _stats_bwd(Kf[f], Vf[f], bf[f], dA, dW)
    out = dict(dq=dq.reshape(L, dk), dk=dk_.reshape(L, dk), dv=dv_.reshape(L, dv),
               dbeta=dbeta.reshape(L), dg_l=dg.reshape(L), dalpha=dalpha, dgamma=dgamma)
    if has_text:
        dW_T = X_T.T @ dS_text
        dA_T = -X_T.T @ (dS_text @ W_T.T) @ X_T.T
        out["dk_text"], out["dv_text"], out["dbeta_text"] = _stats_bwd(kt, vt, bt, dA_T, dW_T)
    else:
        T_ = 0 if k_text is None else len(k_text)
        out["dk_text"], out["dv_text"], out["dbeta_text"] = (np.zeros((T_, dk)), np.zeros((T_, dv)),
                                                             np.zeros(T_))
    return out


def _stats_bwd(K, V, b, dA, dW):
    """Adjoint of A = K^T diag(b) K, W = K^T diag(b) V: returns (dK, dV, db)."""
    dK = b[:, None] * (K @ (dA + dA.T) + V @ dW.T)
    dV = b[:, None] * (K @ dW)
    db = np.einsum("nk,kj,nj->n", K, dA, K) + np.einsum("nk,kj,nj->n", K, dW, V)
    return dK, dV, db


def vda_bwd(inp: dict, dOhat_l, p: O.Params = O.DEFAULT, heads=None):
    """linear_branch_bwd over stacked inputs.

    inp as for vdn_oracle.vdn_attn; dOhat_l: [B, L, H, dv] (the layout of the
    branch output).  heads: optional list of (b, h) to evaluate (others stay
    zero).  Returns a dict of [B, H, ...] arrays and dgamma summed over heads.
    """
    q = inp["q"]
    B, H, L, dk = q.shape
    dv = inp["v"].shape[-1]
    F = inp["alpha"].shape[2]
    T_ = inp["k_text"].shape[2]
    out = dict(dq=np.zeros((B, H, L, dk)), dk=np.zeros((B, H, L, dk)), dv=np.zeros((B, H, L, dv)),
               dbeta=np.zeros((B, H, L)), dg_l=np.zeros((B, H, L)), dalpha=np.zeros((B, H, F, dk)),
               dk_text=np.zeros((B, H, T_, dk)), dv_text=np.zeros((B, H, T_, dv)),
               dbeta_text=np.zeros((B, H, T_)), dgamma=np.zeros(dv))
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in heads:
        r = linear_branch_bwd(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], inp["beta"][b, h],
                              inp["alpha"][b, h], inp["k_text"][b, h], inp["v_text"][b, h],
                              inp["beta_text"][b, h], inp["g_l"][b, h], inp.get("gamma"),
                              np.asarray(dOhat_l)[b, :, h], p)
        for key, val in r.items():
            if key == "dgamma":
                out[key] += val
            else:
                out[key][b, h] = val
    return out
