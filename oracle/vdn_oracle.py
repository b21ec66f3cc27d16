"""Video DeltaNet (VDN) attention forward -- CPU fp64 oracle.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain definition that the
HIP library is checked against.  Only the test-suite, the smoke entry point
and the benchmark's CPU-baseline leg may import it; the product path (the
C-ABI library and its Python binding) never calls it and shares no code with
it.

Source: "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation" (arXiv 2609.20744; page papers.paperslantern.ai).  The extracted
page lost all display math, so every formula below is restated from the
surrounding prose; each function names the passage it follows.  Where the
prose leaves a step open, the reading taken is stated in the docstring.

Notation, per batch b and head h:
  frames f = 0..F-1, N tokens per frame, token row l = f*N + n (frame-major);
  Q_f, K_f in R^{N x dk}, V_f in R^{N x dv};  beta_f in [0,1]^N (write gate);
  alpha_f in (0,1]^{dk} (channel-wise decay gate, one per frame);
  state S in R^{dk x dv}, read out as o = q^T S.

Everything is computed in float64 from the (already rounded) inputs.  No
blocking, fusion or reordering beyond what the definitions state.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# --------------------------------------------------------------------------
# Parameters
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Params:
    """Operator hyper-parameters.

    chunk_frames / window_chunks / anchors: method, local Softmax window --
      the VAE decodes 5 latent frames as one temporal chunk; a query chunk
      sees itself and its preceding and following chunk; the first and last
      latent frames are boundary anchors with four-way connectivity.
    softmax_scale: not printed on the page; the standard 1/sqrt(dk) is taken.
    rms_eps: not printed; 1e-6 is taken.
    text_init_scale: each directional scan starts from this multiple of the
      text state.  The page says the two readouts together count the prompt
      exactly once, which fixes the reading 1/2.
    text_softmax: False (the default) is the video-to-video operator: the
      Softmax branch sees video keys only.  True adds the T text tokens to
      the key set of every video query, always visible, in the same
      normalisation (method, bidirectional linear attention: the text stays
      directly visible to the Softmax branch while the linear memory also
      starts from its summary).  Reading: the text keys join the one softmax
      of each query (not a separate, separately normalised attention), and
      anchor frames see them as well.
    """
    chunk_frames: int = 5
    window_chunks: int = 1
    anchors: bool = True
    softmax_scale: float | None = None     # None -> 1/sqrt(dk)
    rms_eps: float = 1e-6
    text_init_scale: float = 0.5
    text_softmax: bool = False


DEFAULT = Params()


# --------------------------------------------------------------------------
# Frame roles: Softmax visibility and the two linear-attention regions
# --------------------------------------------------------------------------
def chunk_of(f: int, p: Params = DEFAULT) -> int:
    """Temporal chunk of latent frame f (method, local Softmax window)."""
    return f // p.chunk_frames


def is_anchor(f: int, F: int, p: Params = DEFAULT) -> bool:
    """Boundary anchors are the first and the last latent frame."""
    return bool(p.anchors) and (f == 0 or f == F - 1)


def visible_frames(t: int, F: int, p: Params = DEFAULT) -> set[int]:
    """Key frames that query frame t reaches through Softmax.

    Method, local Softmax window and boundary anchors: a query chunk attends
    to itself and its immediately preceding and following chunks (clipped at
    the sequence ends); every frame attends to all tokens of the first and
    last latent frame; those two frames attend to the whole sequence.  The
    result is a set: an anchor that already lies in the window is counted
    once.
    """
    if is_anchor(t, F, p):
        return set(range(F))
    c = chunk_of(t, p)
    vis = {f for f in range(F) if abs(chunk_of(f, p) - c) <= p.window_chunks}
    if p.anchors:
        vis |= {0, F - 1}
    return vis


def visibility(F: int, p: Params = DEFAULT) -> np.ndarray:
    """[F, F] uint8 frame mask, row = query frame, column = key frame."""
    m = np.zeros((F, F), dtype=np.uint8)
    for t in range(F):
        for f in visible_frames(t, F, p):
            m[t, f] = 1
    return m


def window_bounds(t: int, F: int, p: Params = DEFAULT) -> tuple[int, int]:
    """First and last frame of query frame t's local window (anchors aside)."""
    c = chunk_of(t, p)
    lo = max(c - p.window_chunks, 0) * p.chunk_frames
    hi = min((c + p.window_chunks + 1) * p.chunk_frames, F) - 1
    return lo, hi


def linear_regions(t: int, F: int, p: Params = DEFAULT) -> tuple[set[int], set[int]]:
    """Frames written into the forward and the reverse state seen by frame t.

    Method, bidirectional linear attention: the forward state summarises the
    frames before t's Softmax window, the reverse state the frames after it;
    boundary anchors are excluded from both because Softmax already covers
    them.  An anchor query frame already sees every frame through Softmax, so
    both of its regions are empty (reading: its linear memory is text only).
    """
    if is_anchor(t, F, p):
        return set(), set()
    lo, hi = window_bounds(t, F, p)
    fwd = {f for f in range(0, lo) if not is_anchor(f, F, p)}
    rev = {f for f in range(hi + 1, F) if not is_anchor(f, F, p)}
    return fwd, rev


def scan_indices(F: int, p: Params = DEFAULT):
    """Where each query frame reads the chunk-boundary states, and its bridge.

    Method, system section, chunk-wise scans: memory is only read at chunk
    boundaries.  P_fwd[i] is the forward state after chunks 0..i-1 and
    P_rev[i] the reverse state after chunks C-1..i.  Query frame t reads
    P_fwd[i_fwd[t]] and decays it over frames ws[t]..t (the decay bridge
    over the skipped local span); likewise P_rev[i_rev[t]] over t..we[t].
    Returns four int32 arrays of length F.
    """
    C = -(-F // p.chunk_frames)
    i_fwd = np.zeros(F, np.int32)
    ws = np.zeros(F, np.int32)
    i_rev = np.zeros(F, np.int32)
    we = np.zeros(F, np.int32)
    for t in range(F):
        if is_anchor(t, F, p):
            i_fwd[t], ws[t], i_rev[t], we[t] = 0, 0, C, F - 1
            continue
        c = chunk_of(t, p)
        i_fwd[t] = max(c - p.window_chunks, 0)
        ws[t] = i_fwd[t] * p.chunk_frames
        i_rev[t] = min(c + p.window_chunks + 1, C)
        we[t] = min(i_rev[t] * p.chunk_frames, F) - 1
    return i_fwd, ws, i_rev, we


# --------------------------------------------------------------------------
# Video Delta Attention: per-frame statistics and the joint frame update
# --------------------------------------------------------------------------
def frame_stats(K: np.ndarray, V: np.ndarray, beta: np.ndarray):
    """Frame statistics A = K^T B K (key correlations) and W = K^T B V
    (value-key writes), B = diag(beta).

    Video Delta Attention section, the paragraph that stacks a frame's keys
    and values and defines the two frame statistics.
    """
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    b = np.asarray(beta, np.float64)
    A = K.T @ (b[:, None] * K)
    W = K.T @ (b[:, None] * V)
    return A, W


def vda_update(S_prev: np.ndarray, K, V, beta, alpha) -> np.ndarray:
    """One VDA frame update from the state S_prev.

    Video Delta Attention section, joint objective: the new state minimises
      1/2 ||S - S~||_F^2 + 1/2 sum_i beta_i ||k_i^T S - v_i^T||^2,
    with S~ = diag(alpha) S_prev the decayed state.  Setting the gradient to
    zero gives the normal equation (I + A) S = S~ + W and the closed form
    S = (I + A)^{-1} (S~ + W); the inverse lives in key-channel space.
    Reading: the decay is channel-wise on the key channels and is applied
    before the write; beta enters the fit term with weight 1 and no
    frame-size factor.
    """
    A, W = frame_stats(K, V, beta)
    dk = A.shape[0]
    S_tilde = np.asarray(alpha, np.float64)[:, None] * np.asarray(S_prev, np.float64)
    return np.linalg.solve(np.eye(dk) + A, S_tilde + W)


def frame_map(K, V, beta, alpha):
    """The VDA update as an affine map S -> T S + U.

    T = (I + A)^{-1} diag(alpha), U = (I + A)^{-1} W: the transition and
    injection terms that the page's small-matrix inverse emits (system
    section, small-matrix inverse).
    """
    A, W = frame_stats(K, V, beta)
    dk = A.shape[0]
    M = np.eye(dk) + A
    T = np.linalg.solve(M, np.diag(np.asarray(alpha, np.float64)))
    U = np.linalg.solve(M, W)
    return T, U


def text_state(K_T, V_T, beta_T, dk: int, dv: int) -> np.ndarray:
    """Text state: all text tokens summarised into one VDA state.

    Method, bidirectional linear attention (the memory is text-aware) and
    system section (the prompt state is a leading virtual frame): one VDA
    update of the zero state with the text tokens, no decay.  With no text
    tokens the state is zero.
    """
    if K_T is None or len(K_T) == 0:
        return np.zeros((dk, dv))
    return vda_update(np.zeros((dk, dv)), K_T, V_T, beta_T, np.ones(dk))


# --------------------------------------------------------------------------
# Linear branch: two directional memories per query frame
# --------------------------------------------------------------------------
def directional_memory_bruteforce(Kf, Vf, betaf, alpha, S_text, p: Params = DEFAULT):
    """M_fwd[t], M_rev[t] by running each query frame's own recurrence.

    For query frame t the forward memory starts from text_init_scale*S_text
    and visits frames 0..t in order: a frame in t's forward region performs
    the VDA update, every other frame (anchors, the window frames up to t)
    only decays, S <- diag(alpha_f) S.  The reverse memory does the same from
    frame F-1 down to t with the reverse region.
    Reading: excluded frames decay but do not write (the page's accumulated
    channel-wise decay across the skipped span), and the bridge includes the
    query frame's own decay.
    Kf, Vf: [F, N, d]; betaf [F, N]; alpha [F, dk].  Cost O(F^2) updates --
    for small self-test cases only.
    """
    F = Kf.shape[0]
    dk, dv = Kf.shape[2], Vf.shape[2]
    S0 = p.text_init_scale * S_text
    M_fwd = np.zeros((F, dk, dv))
    M_rev = np.zeros((F, dk, dv))
    for t in range(F):
        fwd, rev = linear_regions(t, F, p)
        S = S0.copy()
        for f in range(0, t + 1):
            if f in fwd:
                S = vda_update(S, Kf[f], Vf[f], betaf[f], alpha[f])
            else:
                S = alpha[f][:, None] * S
        M_fwd[t] = S
        S = S0.copy()
        for f in range(F - 1, t - 1, -1):
            if f in rev:
                S = vda_update(S, Kf[f], Vf[f], betaf[f], alpha[f])
            else:
                S = alpha[f][:, None] * S
        M_rev[t] = S
    return M_fwd, M_rev


def frame_maps(Kf, Vf, betaf, alpha, p: Params = DEFAULT):
    """(T_f, U_f) for every frame, with anchor frames masked to decay only
    (T = diag(alpha_f), U = 0): the per-frame elements of the scans."""
    F = Kf.shape[0]
    dk, dv = Kf.shape[2], Vf.shape[2]
    T = np.zeros((F, dk, dk))
    U = np.zeros((F, dk, dv))
    for f in range(F):
        if is_anchor(f, F, p):
            T[f] = np.diag(np.asarray(alpha[f], np.float64))
        else:
            T[f], U[f] = frame_map(Kf[f], Vf[f], betaf[f], alpha[f])
    return T, U


def scan_states(Kf, Vf, betaf, alpha, S_text, p: Params = DEFAULT):
    """Chunk-boundary states of the forward and reverse frame recurrences.

    Method (bidirectional scans) and system section (chunk-wise scans keep
    the boundary states): with anchors masked to decay only,
      forward  S_f = T_f S_{f-1} + U_f from S_{-1} = text_init_scale*S_text,
      reverse  S_f = T_f S_{f+1} + U_f from S_F  = text_init_scale*S_text.
    P_fwd[i] = forward state after frames 0..i*cf-1 (i = 0..C);
    P_rev[i] = reverse state after frames F-1..i*cf (i = 0..C).
    Run frame by frame -- no chunk composition.
    """
    F = Kf.shape[0]
    cf = p.chunk_frames
    C = -(-F // cf)
    T, U = frame_maps(Kf, Vf, betaf, alpha, p)
    S0 = p.text_init_scale * S_text
    dk, dv = S0.shape
    P_fwd = np.zeros((C + 1, dk, dv))
    P_rev = np.zeros((C + 1, dk, dv))
    S = S0.copy()
    P_fwd[0] = S
    for f in range(F):
        S = T[f] @ S + U[f]
        if (f + 1) % cf == 0 or f == F - 1:
            P_fwd[-(-(f + 1) // cf)] = S
    S = S0.copy()
    P_rev[C] = S
    for f in range(F - 1, -1, -1):
        S = T[f] @ S + U[f]
        if f % cf == 0:
            P_rev[f // cf] = S
    return P_fwd, P_rev


def directional_memory_scan(P_fwd, P_rev, alpha, p: Params = DEFAULT):
    """M_fwd[t], M_rev[t] from the chunk-boundary states (gather + bridge).

    Method, bidirectional linear attention: at readout time gather the state
    just outside the window boundary and apply the accumulated channel-wise
    decay across the skipped local span:
      M_fwd[t] = diag(prod_{f=ws..t} alpha_f) P_fwd[i_fwd[t]],
      M_rev[t] = diag(prod_{f=t..we} alpha_f) P_rev[i_rev[t]].
    """
    F = alpha.shape[0]
    i_fwd, ws, i_rev, we = scan_indices(F, p)
    dk, dv = P_fwd.shape[1:]
    M_fwd = np.zeros((F, dk, dv))
    M_rev = np.zeros((F, dk, dv))
    a = np.asarray(alpha, np.float64)
    for t in range(F):
        d_f = np.prod(a[ws[t]:t + 1], axis=0)
        d_r = np.prod(a[t:we[t] + 1], axis=0)
        M_fwd[t] = d_f[:, None] * P_fwd[i_fwd[t]]
        M_rev[t] = d_r[:, None] * P_rev[i_rev[t]]
    return M_fwd, M_rev


def rms_norm(x: np.ndarray, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: gamma * x / sqrt(mean(x^2) + eps).
    Method, branch calibration: the linear readout is RMS-normalised.
    Reading: per (token, head) over dv."""
    x = np.asarray(x, np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    g = 1.0 if gamma is None else np.asarray(gamma, np.float64)
    return g * x / r


def linear_branch(Q, M_fwd, M_rev, g_l, gamma, p: Params = DEFAULT):
    """O_l = q^T (M_fwd[t] + M_rev[t]) per token; gated output
    Ohat_l = g_l * RMSNorm(O_l).

    Method: the distant-context output is the sum of the two readouts; the
    linear readout is RMS-normalised and passed through its own output gate.
    Q: [F, N, dk]; g_l: [F, N] (post-sigmoid).  Returns (O_l, Ohat_l) as
    [F, N, dv].
    """
    Q = np.asarray(Q, np.float64)
    M = M_fwd + M_rev
    O_l = np.einsum("fnk,fkv->fnv", Q, M)
    Ohat = np.asarray(g_l, np.float64)[..., None] * rms_norm(O_l, gamma, p.rms_eps)
    return O_l, Ohat


# --------------------------------------------------------------------------
# Softmax branch
# --------------------------------------------------------------------------
def softmax_rows(Qrows, t, Kf, Vf, p: Params = DEFAULT, K_text=None, V_text=None):
    """Softmax attention of query rows of frame t over Vis(t).

    Method, local Softmax window: exact Softmax attention over the tokens of
    every visible key frame (each frame once).  With p.text_softmax the T
    text tokens (K_text [T, dk], V_text [T, dv]) are further keys of the
    same softmax, visible to every query.  Scale 1/sqrt(dk) unless given.
    Returns (O [n, dv], lse [n]) with lse the natural-log normaliser of the
    scaled logits.
    """
    F = Kf.shape[0]
    dk = Kf.shape[2]
    scale = (1.0 / math.sqrt(dk)) if p.softmax_scale is None else p.softmax_scale
    fr = sorted(visible_frames(t, F, p))
    blocks_k = [np.asarray(Kf[f], np.float64) for f in fr]
    blocks_v = [np.asarray(Vf[f], np.float64) for f in fr]
    if p.text_softmax and K_text is not None and len(K_text):
        blocks_k.append(np.asarray(K_text, np.float64))
        blocks_v.append(np.asarray(V_text, np.float64))
    Kv = np.concatenate(blocks_k)
    Vv = np.concatenate(blocks_v)
    s = (np.asarray(Qrows, np.float64) @ Kv.T) * scale
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    O = (e / z) @ Vv
    lse = (m + np.log(z))[:, 0]
    return O, lse


def softmax_branch(Qf, Kf, Vf, g_s, p: Params = DEFAULT, K_text=None, V_text=None):
    """O_s and Ohat_s = g_s * O_s for every token of one head.

    Method, branch calibration: a content-dependent sigmoid gate scales the
    Softmax readout (the gate values are inputs here).
    Qf, Kf, Vf: [F, N, d]; g_s: [F, N]; K_text, V_text: [T, d] (used only
    with p.text_softmax).  Returns (O_s, Ohat_s, lse).
    """
    F, N = Qf.shape[:2]
    dv = Vf.shape[2]
    O = np.zeros((F, N, dv))
    lse = np.zeros((F, N))
    for t in range(F):
        O[t], lse[t] = softmax_rows(Qf[t], t, Kf, Vf, p, K_text, V_text)
    return O, np.asarray(g_s, np.float64)[..., None] * O, lse


# --------------------------------------------------------------------------
# Merge
# --------------------------------------------------------------------------
def merge(Ohat_s, Ohat_l, W_s=None, W_l=None):
    """out = Ohat_s W_s + Ohat_l W_l over the concatenated heads.

    Method, branch calibration: each branch has its own output projection;
    the two projected outputs are added.  Ohat_*: [B, L, H, dv] (token-major,
    heads concatenated as h*dv + j); W_*: [H*dv, D].  With W_s = W_l = None
    the projections are identity and out = Ohat_s + Ohat_l, [B, L, H, dv].
    """
    Ohat_s = np.asarray(Ohat_s, np.float64)
    Ohat_l = np.asarray(Ohat_l, np.float64)
    if W_s is None and W_l is None:
        return Ohat_s + Ohat_l
    B, L, H, dv = Ohat_s.shape
    xs = Ohat_s.reshape(B, L, H * dv)
    xl = Ohat_l.reshape(B, L, H * dv)
    return xs @ np.asarray(W_s, np.float64) + xl @ np.asarray(W_l, np.float64)


# --------------------------------------------------------------------------
# One head and the whole operator
# --------------------------------------------------------------------------
def vdn_head(q, k, v, beta, alpha, k_text, v_text, beta_text, g_s, g_l,
             gamma=None, p: Params = DEFAULT, F: int | None = None,
             linear_form: str = "scan", want_softmax: bool = True):
    """Every intermediate of the operator for one (b, h).

    q, k, v: [L, d] frame-major; beta, g_s, g_l: [L]; alpha: [F, dk];
    k_text, v_text: [T, d]; beta_text: [T].
    linear_form: "scan" (chunk-boundary states + gather/bridge) or
    "bruteforce" (each query frame's own masked recurrence).
    """
    L, dk = q.shape
    dv = v.shape[1]
    F = alpha.shape[0] if F is None else F
    N = L // F
    Qf = np.asarray(q, np.float64).reshape(F, N, dk)
    Kf = np.asarray(k, np.float64).reshape(F, N, dk)
    Vf = np.asarray(v, np.float64).reshape(F, N, dv)
    bf = np.asarray(beta, np.float64).reshape(F, N)
    a = np.asarray(alpha, np.float64)
    S_text = text_state(k_text, v_text, beta_text, dk, dv)
    out = {"S_text": S_text}
    if linear_form == "scan":
        P_fwd, P_rev = scan_states(Kf, Vf, bf, a, S_text, p)
        M_fwd, M_rev = directional_memory_scan(P_fwd, P_rev, a, p)
        out["P_fwd"], out["P_rev"] = P_fwd, P_rev
    elif linear_form == "bruteforce":
        M_fwd, M_rev = directional_memory_bruteforce(Kf, Vf, bf, a, S_text, p)
    else:
        raise ValueError(linear_form)
    out["M_fwd"], out["M_rev"] = M_fwd, M_rev
    O_l, Ohat_l = linear_branch(Qf, M_fwd, M_rev, np.reshape(g_l, (F, N)), gamma, p)
    out["O_l"], out["Ohat_l"] = O_l.reshape(L, dv), Ohat_l.reshape(L, dv)
    if want_softmax:
        O_s, Ohat_s, lse = softmax_branch(Qf, Kf, Vf, np.reshape(g_s, (F, N)), p, k_text, v_text)
        out["O_s"], out["Ohat_s"], out["lse"] = (O_s.reshape(L, dv),
                                                 Ohat_s.reshape(L, dv), lse.reshape(L))
    return out


def vdn_attn(inp: dict, p: Params = DEFAULT, linear_form: str = "scan"):
    """The whole operator on stacked inputs.

    inp holds numpy arrays: q, k, v [B,H,L,d]; beta, g_s, g_l [B,H,L];
    alpha [B,H,F,dk]; k_text, v_text [B,H,T,d]; beta_text [B,H,T];
    optional gamma [dv], W_s, W_l [H*dv, D].
    Returns a dict with per-head intermediates stacked on [B,H,...] and
    "out" ([B,L,D], or [B,L,H,dv] without projections).
    """
    q = inp["q"]
    B, H, L, dk = q.shape
    dv = inp["v"].shape[-1]
    F = inp["alpha"].shape[2]
    heads = {}
    for b in range(B):
        for h in range(H):
            r = vdn_head(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                         inp["beta"][b, h], inp["alpha"][b, h],
                         inp["k_text"][b, h], inp["v_text"][b, h], inp["beta_text"][b, h],
                         inp["g_s"][b, h], inp["g_l"][b, h], inp.get("gamma"),
                         p, F, linear_form)
            for key, val in r.items():
                heads.setdefault(key, np.zeros((B, H) + val.shape))[b, h] = val
    Ohat_s = heads["Ohat_s"].transpose(0, 2, 1, 3)   # [B, L, H, dv]
    Ohat_l = heads["Ohat_l"].transpose(0, 2, 1, 3)
    heads["out"] = merge(Ohat_s, Ohat_l, inp.get("W_s"), inp.get("W_l"))
    return heads


def head_rows(q, k, v, beta, alpha, k_text, v_text, beta_text, g_s, g_l, rows,
              gamma=None, p: Params = DEFAULT, want_softmax: bool = True):
    """The same per-head definitions evaluated only at the token rows `rows`
    (frame-major indices), for checks at sizes where every row is too slow.

    The chunk-boundary states are computed in full (they are O(F) updates);
    the Softmax and linear readouts only for the chosen rows.  Returns a
    dict with S_text, P_fwd, P_rev and, per chosen row, O_s, Ohat_s, lse,
    O_l, Ohat_l.
    """
    L, dk = q.shape
    dv = v.shape[1]
    F = alpha.shape[0]
    N = L // F
    rows = np.asarray(rows, np.int64)
    Kf = np.asarray(k, np.float64).reshape(F, N, dk)
    Vf = np.asarray(v, np.float64).reshape(F, N, dv)
    bf = np.asarray(beta, np.float64).reshape(F, N)
    a = np.asarray(alpha, np.float64)
    S_text = text_state(k_text, v_text, beta_text, dk, dv)
    P_fwd, P_rev = scan_states(Kf, Vf, bf, a, S_text, p)
    M_fwd, M_rev = directional_memory_scan(P_fwd, P_rev, a, p)
    n = len(rows)
    out = {"S_text": S_text, "P_fwd": P_fwd, "P_rev": P_rev,
           "O_l": np.zeros((n, dv)), "Ohat_l": np.zeros((n, dv))}
    if want_softmax:
        out.update(O_s=np.zeros((n, dv)), Ohat_s=np.zeros((n, dv)), lse=np.zeros(n))
    frames = rows // N
    for t in np.unique(frames):
        sel = np.nonzero(frames == t)[0]
        qr = np.asarray(q, np.float64)[rows[sel]]
        O_l, Oh_l = linear_branch(qr[None], M_fwd[t][None], M_rev[t][None],
                                  np.asarray(g_l, np.float64)[rows[sel]][None], gamma, p)
        out["O_l"][sel], out["Ohat_l"][sel] = O_l[0], Oh_l[0]
        if want_softmax:
            O_s, lse = softmax_rows(qr, int(t), Kf, Vf, p, k_text, v_text)
            out["O_s"][sel] = O_s
            out["Ohat_s"][sel] = np.asarray(g_s, np.float64)[rows[sel]][:, None] * O_s
            out["lse"][sel] = lse
    return out


# --------------------------------------------------------------------------
# Algorithmic work counts (used for reporting only)
# --------------------------------------------------------------------------
def visible_pairs(F: int, p: Params = DEFAULT) -> int:
    """Number of visible (query frame, key frame) pairs."""
    return int(visibility(F, p).sum())
