"""Backward pass of the merge (separate output projections summed) -- CPU
fp64 oracle.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and shares no code with it.

Source: "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation".  Method, branch calibration: each branch has its own output
projection and the projected outputs are added,
  out = Ohat_s W_s + Ohat_l W_l            (tokens x heads*d_v) (heads*d_v x D),
and the experiments train through the layer.  The page prints no gradients;
those of a sum of two matrix products are, for an output gradient dout,
  dOhat_s = dout W_s^T,  dOhat_l = dout W_l^T,
  dW_s = Ohat_s^T dout,  dW_l = Ohat_l^T dout,
and without projections (out = Ohat_s + Ohat_l) dOhat_s = dOhat_l = dout.
Everything in float64.
"""
from __future__ import annotations

import numpy as np


def merge_bwd(Ohat_s, Ohat_l, W_s, W_l, dout):
    """Ohat_s, Ohat_l: [M, K]; W_s, W_l: [K, D] or both None; dout: [M, D].
    Returns (dOhat_s, dOhat_l, dW_s, dW_l) (dW_* None without projections)."""
    dout = np.asarray(dout, np.float64)
    if W_s is None:
        return dout.copy(), dout.copy(), None, None
    Os, Ol, Ws, Wl = (np.asarray(x, np.float64) for x in (Ohat_s, Ohat_l, W_s, W_l))
    return dout @ Ws.T, dout @ Wl.T, Os.T @ dout, Ol.T @ dout
