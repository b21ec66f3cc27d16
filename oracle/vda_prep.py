"""VDA-Prep, the linear branch's feature map -- CPU fp64 oracle.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and shares no code with it.

Source: "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation" (arXiv 2609.20744).  Method section, the two branches: the linear
branch applies its own feature map to the projected inputs -- a separable
short convolution on K and V made of a depthwise spatial filter and a
five-tap temporal filter, followed by SiLU, with L2 normalisation on Q and K,
and no rotary embedding.  System section, fused VDA kernels: VDA-Prep fuses
the temporal convolution, SiLU, L2 normalisation and the conversion to the
frame-major layout for K and V.

Readings where the page is silent (each also listed in the design notes):
  * spatial filter size: not printed -- a parameter (kernel_h x kernel_w, odd),
    default 3 x 3;
  * temporal alignment: not printed -- centred taps (offsets -2..+2 for five
    taps) by default, causal taps (offsets -4..0) as an option; the scans of
    this operator run in both directions, which the centred reading matches;
  * padding: zeros outside the clip (frames) and outside the latent grid;
  * no bias terms; one filter per channel (depthwise, per head);
  * order: SiLU after the full separable convolution; L2 normalisation of K
    after SiLU; Q is L2-normalised only (no convolution, no SiLU);
  * L2 normalisation: x / sqrt(sum(x^2) + eps) over the d channels of one
    token of one head, eps = 1e-6;
  * layouts: inputs token-major [B, L, H, d] (the projection output), outputs
    frame-major [B, H, L, d] with L = F * N, token n = y * grid_w + x.

Everything is computed in float64 from the (already rounded) inputs.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class PrepParams:
    grid_h: int
    grid_w: int
    kernel_h: int = 3
    kernel_w: int = 3
    taps: int = 5
    causal: bool = False
    l2_eps: float = 1e-6

    @property
    def t0(self) -> int:
        """Index of the tap that multiplies the output's own frame."""
        return self.taps - 1 if self.causal else (self.taps - 1) // 2


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def l2_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def short_conv(x: np.ndarray, w_sp: np.ndarray, w_t: np.ndarray, p: PrepParams) -> np.ndarray:
    """Separable depthwise convolution of one head's features.

    x: [F, grid_h, grid_w, d]; w_sp: [d, kernel_h, kernel_w]; w_t: [d, taps].
    out[f, y, x, c] = sum_tau w_t[c, tau] sum_{dy,dx} w_sp[c, dy, dx]
                      * x[f + tau - t0, y + dy - ry, x + dx - rx, c],
    with ry = (kernel_h - 1) / 2, rx = (kernel_w - 1) / 2 and zeros outside.
    """
    F, Hs, Ws, d = x.shape
    kh, kw, taps = p.kernel_h, p.kernel_w, p.taps
    ry, rx, t0 = (kh - 1) // 2, (kw - 1) // 2, p.t0
    xp = np.zeros((F + taps - 1, Hs + kh - 1, Ws + kw - 1, d))
    xp[t0:t0 + F, ry:ry + Hs, rx:rx + Ws, :] = x
    out = np.zeros((F, Hs, Ws, d))
    for tau in range(taps):
        for dy in range(kh):
            for dx in range(kw):
                out += (w_t[:, tau] * w_sp[:, dy, dx]) * xp[tau:tau + F, dy:dy + Hs, dx:dx + Ws, :]
    return out


def prep_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, w_sp: np.ndarray, w_t: np.ndarray,
              p: PrepParams):
    """Feature map of one (batch, head): q, k, v [L, d] frame-major token rows.

    Returns (q', k', v'), each [L, d]:
      q' = L2(q),  k' = L2(SiLU(conv(k))),  v' = SiLU(conv(v)).
    """
    L, d = k.shape
    N = p.grid_h * p.grid_w
    F = L // N
    shape = (F, p.grid_h, p.grid_w, d)
    kc = silu(short_conv(k.reshape(shape), w_sp, w_t, p)).reshape(L, d)
    vc = silu(short_conv(v.reshape(shape), w_sp, w_t, p)).reshape(L, d)
    return l2_normalize(q, p.l2_eps), l2_normalize(kc, p.l2_eps), vc


def vda_prep(q: np.ndarray, k: np.ndarray, v: np.ndarray, w_sp: np.ndarray, w_t: np.ndarray,
             p: PrepParams):
    """Whole batch: q, k, v [B, L, H, d] token-major; w_sp [H, d, kh, kw]; w_t [H, d, taps].

    Returns q', k', v' [B, H, L, d] (frame-major, head-major).
    """
    B, L, H, d = q.shape
    outs = [np.zeros((B, H, L, d)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            r = prep_head(np.asarray(q[b, :, h, :], np.float64), np.asarray(k[b, :, h, :], np.float64),
                          np.asarray(v[b, :, h, :], np.float64), np.asarray(w_sp[h], np.float64),
                          np.asarray(w_t[h], np.float64), p)
            for o, x in zip(outs, r):
                o[b, h] = x
    return tuple(outs)


def prep_rows(k: np.ndarray, v: np.ndarray, w_sp: np.ndarray, w_t: np.ndarray, rows, p: PrepParams):
    """k', v' of one head at the given token rows only (for sampled checks of
    large inputs).  k, v: [L, d] frame-major rows of one head.  The same sum as
    `short_conv`, taken over each row's neighbourhood."""
    L, d = k.shape
    N = p.grid_h * p.grid_w
    F = L // N
    kh, kw, taps = p.kernel_h, p.kernel_w, p.taps
    ry, rx, t0 = (kh - 1) // 2, (kw - 1) // 2, p.t0
    ko = np.zeros((len(rows), d))
    vo = np.zeros((len(rows), d))
    for i, l in enumerate(rows):
        f, n = divmod(int(l), N)
        y, x = divmod(n, p.grid_w)
        for tau in range(taps):
            fs = f + tau - t0
            if not 0 <= fs < F:
                continue
            for dy in range(kh):
                ys = y + dy - ry
                if not 0 <= ys < p.grid_h:
                    continue
                for dx in range(kw):
                    xs = x + dx - rx
                    if not 0 <= xs < p.grid_w:
                        continue
                    src = fs * N + ys * p.grid_w + xs
                    wgt = w_t[:, tau] * w_sp[:, dy, dx]
                    ko[i] += wgt * k[src]
                    vo[i] += wgt * v[src]
    return l2_normalize(silu(ko), p.l2_eps), silu(vo)
