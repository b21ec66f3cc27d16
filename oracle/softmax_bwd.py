"""Backward pass of the window + anchor Softmax branch -- CPU fp64 oracle.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and shares no code with it.

Source: "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation" (arXiv 2609.20744).  Method, local Softmax window and branch
calibration, defines the forward: for query frame t,
  O_s[t] = softmax(scale * Q_t K_vis^T) V_vis,   Ohat_s = g_s * O_s,
with K_vis, V_vis the tokens of the visible key frames Vis(t), each frame
once.  The experiments section trains the model through this operator (the
staged adaptation), which needs its gradients; the page prints none, so they
are the chain rule applied to that definition, written out per query frame:
  dO  = g_s * dOhat                     (gradient of the ungated output)
  dg  = rowsum(dOhat * O_s)
  P   = softmax(scale * Q_t K_vis^T)
  dV_vis += P^T dO
  dP  = dO V_vis^T
  dS  = P * (dP - rowsum(dO * O_s))
  dQ_t = scale * dS K_vis,   dK_vis += scale * dS^T Q_t
Contributions to the keys and values of a frame are summed over every query
frame that sees it.  With the text-keys option (method, bidirectional linear
attention: the text stays visible to the Softmax branch) the T text tokens
are further keys of every query frame, in the same softmax; their gradients
are summed over all query frames.  Everything in float64.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import vdn_oracle as O


def softmax_branch_bwd(Qf, Kf, Vf, g_s, dOhat, p: O.Params = O.DEFAULT, K_text=None,
                       V_text=None):
    """Gradients of the gated Softmax branch for one head.

    Qf, Kf, Vf: [F, N, d]; g_s: [F, N] (post-sigmoid gate values, an input);
    dOhat: [F, N, dv] the gradient of Ohat_s.  Returns (dQ, dK, dV, dg) with
    the shapes of Qf, Kf, Vf and g_s; with p.text_softmax and K_text, V_text
    [T, d] given, (dQ, dK, dV, dg, dK_text, dV_text).
    """
    Qf = np.asarray(Qf, np.float64)
    Kf = np.asarray(Kf, np.float64)
    Vf = np.asarray(Vf, np.float64)
    g = np.asarray(g_s, np.float64)
    dOh = np.asarray(dOhat, np.float64)
    F, N, dk = Qf.shape
    scale = (1.0 / math.sqrt(dk)) if p.softmax_scale is None else p.softmax_scale
    text = bool(p.text_softmax) and K_text is not None
    Kt = np.asarray(K_text, np.float64).reshape(-1, dk) if text else np.zeros((0, dk))
    Vt = np.asarray(V_text, np.float64).reshape(-1, Vf.shape[2]) if text else np.zeros((0, Vf.shape[2]))
    dQ = np.zeros_like(Qf)
    dK = np.zeros_like(Kf)
    dV = np.zeros_like(Vf)
    dg = np.zeros((F, N))
    dKt = np.zeros_like(Kt)
    dVt = np.zeros_like(Vt)
    for t in range(F):
        fr = sorted(O.visible_frames(t, F, p))
        Kv = np.concatenate([Kf[f] for f in fr] + [Kt])
        Vv = np.concatenate([Vf[f] for f in fr] + [Vt])
        s = scale * (Qf[t] @ Kv.T)
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        Os = P @ Vv
        dO = g[t][:, None] * dOh[t]
        dg[t] = np.sum(dOh[t] * Os, axis=1)
        dVv = P.T @ dO
        dP = dO @ Vv.T
        dS = P * (dP - np.sum(dO * Os, axis=1, keepdims=True))
        dQ[t] = scale * (dS @ Kv)
        dKv = scale * (dS.T @ Qf[t])
        for i, f in enumerate(fr):
            dK[f] += dKv[i * N:(i + 1) * N]
            dV[f] += dVv[i * N:(i + 1) * N]
        dKt += dKv[len(fr) * N:]
        dVt += dVv[len(fr) * N:]
    if text:
        return dQ, dK, dV, dg, dKt, dVt
    return dQ, dK, dV, dg


def softmax_bwd_rows(q, k, v, g_s, dOhat, F: int, qrows, kframe: int | None, krows,
                     p: O.Params = O.DEFAULT, K_text=None, V_text=None):
    """The same gradients at chosen rows only, for checks at sizes where the
    whole backward is too slow.  q, k, v, dOhat: [L, d] frame-major rows of
    one head; g_s: [L].  Returns (dQ at qrows, dK and dV at krows, which must
    all lie in frame kframe).  dK/dV need every query frame that sees
    kframe in full (for their normalisers and Dq); by symmetry of the
    visibility those are visible_frames(kframe).  With p.text_softmax the
    text keys K_text, V_text [T, d] join every query frame's keys (they
    enter dQ and every normaliser; their own gradients are not evaluated
    here)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g_s, np.float64)
    dOh = np.asarray(dOhat, np.float64)
    L, dk_ = q.shape
    N = L // F
    scale = (1.0 / math.sqrt(dk_)) if p.softmax_scale is None else p.softmax_scale
    Qf, Kf, Vf = (x.reshape(F, N, -1) for x in (q, k, v))
    text = bool(p.text_softmax) and K_text is not None
    Kt = np.asarray(K_text, np.float64).reshape(-1, dk_) if text else np.zeros((0, dk_))
    Vt = np.asarray(V_text, np.float64).reshape(-1, v.shape[1]) if text else np.zeros((0, v.shape[1]))

    def frame_terms(t, rows_in_t):
        fr = sorted(O.visible_frames(t, F, p))
        Kv = np.concatenate([Kf[f] for f in fr] + [Kt])
        Vv = np.concatenate([Vf[f] for f in fr] + [Vt])
        Q = Qf[t][rows_in_t]
        s = scale * (Q @ Kv.T)
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        rows = t * N + np.asarray(rows_in_t)
        dO = g[rows][:, None] * dOh[rows]
        Dq = np.sum(dO * (P @ Vv), axis=1, keepdims=True)
        return fr, Kv, Vv, Q, P, dO, Dq

    qrows = np.asarray(qrows, np.int64)
    dQ = np.zeros((len(qrows), dk_))
    for t in np.unique(qrows // N):
        sel = np.nonzero(qrows // N == t)[0]
        fr, Kv, Vv, Q, P, dO, Dq = frame_terms(int(t), qrows[sel] % N)
        dS = P * (dO @ Vv.T - Dq)
        dQ[sel] = scale * (dS @ Kv)
    krows = np.asarray(krows, np.int64)
    dK = np.zeros((len(krows), dk_))
    dV = np.zeros((len(krows), v.shape[1]))
    if len(krows):
        assert np.all(krows // N == kframe)
        for t in sorted(O.visible_frames(kframe, F, p)):
            fr, Kv, Vv, Q, P, dO, Dq = frame_terms(t, np.arange(N))
            col = fr.index(kframe) * N + krows % N      # the sampled keys among t's keys
            Pc = P[:, col]
            dS = Pc * (dO @ v[krows].T - Dq)
            dK += scale * (dS.T @ Q)
            dV += Pc.T @ dO
    return dQ, dK, dV
