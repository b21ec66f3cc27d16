"""Seeded synthetic inputs for the VDN attention operator.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the operator's arithmetic.  Both the HIP path (through its
tests and the benchmark) and the CPU oracle consume exactly the arrays made
here, so the two sides always see the same rounded values.

Every tensor of one (config, b, h) comes from its own stream,
numpy.random.default_rng(SeedSequence([cfg_seed, tensor_id, b, h])), so one
head can be regenerated on its own without drawing the others.

The workloads stand in for MiniMax H3 latents (the page's workload, which is
not available): synthetic tensors with the shapes of the five named
configurations.  Distributions:
  q, v, v_text ~ N(0, 1);  k, k_text ~ N(0, 1) then L2-normalised per token
  (before rounding);  beta, beta_text ~ U(0,1) (tiny) or sigmoid(N(0,1));
  g_s, g_l ~ U(0,1) per (token, head) -- per head and broadcast for the
  H3-scale layer;  alpha (channel-wise decay) ~ U(0.9, 1) per (frame,
  channel), with variants "unit" (all ones) and "u01" (U(0,1));
  W_s, W_l ~ N(0, 1/(H*dv)) with D = H*dv;  gamma = 1.
  The medium configuration copies 5% of its frames from their predecessor
  (frames drawn without replacement from 1..F-1, applied in increasing order)
  to stress correlated writes.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

# tensor ids of the seed sequence
_ID = dict(q=0, k=1, v=2, beta=3, alpha=4, k_text=5, v_text=6, beta_text=7,
           g_s=8, g_l=9, W_s=10, W_l=11, dup=12, prep_q=13, prep_k=14, prep_v=15,
           prep_ws=16, prep_wt=17, d_out=18, d_out_l=19)

# latent grid (rows x columns) of one frame for each configuration, N = rows * columns
GRIDS = {"tiny": (4, 4), "small": (16, 16), "medium": (24, 16), "h3": (48, 32), "long": (32, 24)}


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str          # "f32" or "bf16": storage/compute dtype of q,k,v,text,W,out
    B: int
    H: int
    d: int              # d_k = d_v
    F: int
    N: int
    T: int
    seed: int
    beta: str = "sigmoid"       # "uniform" | "sigmoid" | "zero" (video tokens only)
    gates: str = "token"        # "token" | "head"
    alpha: str = "u0.9"         # "u0.9" | "unit" | "u01"
    dup_frac: float = 0.0
    proj: bool = True           # output projections present (else identity)

    @property
    def L(self) -> int:
        return self.F * self.N

    @property
    def D(self) -> int:
        return self.H * self.d

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "tiny": Config("tiny", "f32", 1, 1, 16, 20, 16, 8, 101, beta="uniform"),
    "small": Config("small", "bf16", 1, 8, 64, 60, 256, 64, 102),
    "medium": Config("medium", "bf16", 1, 16, 128, 100, 384, 512, 103, dup_frac=0.05),
    "h3": Config("h3", "bf16", 1, 24, 128, 120, 1536, 512, 104, gates="head"),
    "long": Config("long", "bf16", 1, 16, 128, 600, 768, 256, 105),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); the
    result is returned as float32 holding exactly representable values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exact bfloat16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _rng(cfg: Config, tid: str, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, _ID[tid], b, h]))


def _store(cfg: Config, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float32)
    return round_bf16(x) if cfg.dtype == "bf16" else x


def _normal(cfg, tid, b, h, shape):
    return _rng(cfg, tid, b, h).standard_normal(shape, dtype=np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _gate01(cfg, tid, b, h, shape):
    g = _rng(cfg, tid, b, h)
    if cfg.gates == "head":
        return np.full(shape, g.random(dtype=np.float32), dtype=np.float32)
    return g.random(shape, dtype=np.float32)


def _beta(cfg, tid, b, h, n):
    g = _rng(cfg, tid, b, h)
    if cfg.beta == "uniform":
        return g.random(n, dtype=np.float32)
    if cfg.beta == "zero" and tid == "beta":   # video write gate only
        return np.zeros(n, np.float32)
    z = g.standard_normal(n, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def _alpha(cfg, b, h):
    g = _rng(cfg, "alpha", b, h)
    shape = (cfg.F, cfg.d)
    if cfg.alpha == "unit":
        return np.ones(shape, np.float32)
    if cfg.alpha == "u01":
        # U(0,1] : 1 - U[0,1)
        return (1.0 - g.random(shape, dtype=np.float64)).astype(np.float32)
    return (0.9 + 0.1 * (1.0 - g.random(shape, dtype=np.float64))).astype(np.float32)


def duplicated_frames(cfg: Config) -> list[int]:
    """Frames f (in increasing order) that are copies of frame f-1."""
    n = int(round(cfg.dup_frac * cfg.F))
    if n <= 0:
        return []
    g = _rng(cfg, "dup")
    return sorted(int(x) for x in g.choice(np.arange(1, cfg.F), size=n, replace=False))


def head_inputs(cfg: Config, b: int, h: int) -> dict:
    """All per-(b, h) inputs as float32 arrays already rounded to cfg.dtype.

    q, k, v: [L, d]; beta, g_s, g_l: [L]; alpha: [F, d] (always float32);
    k_text, v_text: [T, d]; beta_text: [T].
    """
    L, d, T = cfg.L, cfg.d, cfg.T
    out = {
        "q": _store(cfg, _normal(cfg, "q", b, h, (L, d))),
        "k": _store(cfg, _unit_rows(_normal(cfg, "k", b, h, (L, d)))),
        "v": _store(cfg, _normal(cfg, "v", b, h, (L, d))),
        "beta": _beta(cfg, "beta", b, h, L),
        "alpha": _alpha(cfg, b, h),
        "k_text": _store(cfg, _unit_rows(_normal(cfg, "k_text", b, h, (T, d)))),
        "v_text": _store(cfg, _normal(cfg, "v_text", b, h, (T, d))),
        "beta_text": _beta(cfg, "beta_text", b, h, T),
        "g_s": _gate01(cfg, "g_s", b, h, L),
        "g_l": _gate01(cfg, "g_l", b, h, L),
    }
    N = cfg.N
    for f in duplicated_frames(cfg):
        for key in ("q", "k", "v", "beta", "g_s", "g_l"):
            x = out[key]
            x[f * N:(f + 1) * N] = x[(f - 1) * N:f * N]
        out["alpha"][f] = out["alpha"][f - 1]
    return out


def proj_weights(cfg: Config):
    """W_s, W_l [H*d, D] ~ N(0, 1/(H*d)), rounded to cfg.dtype; None, None
    when the configuration has no projections."""
    if not cfg.proj:
        return None, None
    K = cfg.H * cfg.d
    s = np.float32(1.0 / np.sqrt(K))
    ws = _store(cfg, _normal(cfg, "W_s", 0, 0, (K, cfg.D)) * s)
    wl = _store(cfg, _normal(cfg, "W_l", 0, 0, (K, cfg.D)) * s)
    return ws, wl


def full_inputs(cfg: Config, threads: int | None = None) -> dict:
    """Stacked inputs: q, k, v [B,H,L,d]; beta, g_s, g_l [B,H,L];
    alpha [B,H,F,d]; k_text, v_text [B,H,T,d]; beta_text [B,H,T];
    gamma [d]; W_s, W_l [H*d, D] or None.  float32 arrays holding values
    exact in cfg.dtype.  Heads are drawn in parallel threads."""
    B, H = cfg.B, cfg.H
    shapes = {"q": (cfg.L, cfg.d), "k": (cfg.L, cfg.d), "v": (cfg.L, cfg.d),
              "beta": (cfg.L,), "alpha": (cfg.F, cfg.d), "k_text": (cfg.T, cfg.d),
              "v_text": (cfg.T, cfg.d), "beta_text": (cfg.T,), "g_s": (cfg.L,),
              "g_l": (cfg.L,)}
    out = {k: np.empty((B, H) + s, np.float32) for k, s in shapes.items()}

    def one(bh):
        b, h = bh
        r = head_inputs(cfg, b, h)
        for k in shapes:
            out[k][b, h] = r[k]

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with _cf.ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        list(ex.map(one, [(b, h) for b in range(B) for h in range(H)]))
    out["gamma"] = np.ones(cfg.d, np.float32)
    out["W_s"], out["W_l"] = proj_weights(cfg)
    return out


def prep_head_inputs(cfg: Config, b: int, h: int) -> dict:
    """Raw projection outputs of one (b, h) for the linear branch's feature
    map: q, k, v [L, d] frame-major rows ~ N(0, 1), rounded to cfg.dtype."""
    return {key: _store(cfg, _normal(cfg, "prep_" + key, b, h, (cfg.L, cfg.d))) for key in ("q", "k", "v")}


def prep_filters(cfg: Config, kernel_h: int = 3, kernel_w: int = 3, taps: int = 5):
    """Depthwise filters: spatial [H, d, kh, kw] ~ N(0, 1/(kh kw)), temporal
    [H, d, taps] ~ N(0, 1/taps), float32."""
    ws = _rng(cfg, "prep_ws").standard_normal((cfg.H, cfg.d, kernel_h, kernel_w)) / np.sqrt(kernel_h * kernel_w)
    wt = _rng(cfg, "prep_wt").standard_normal((cfg.H, cfg.d, taps)) / np.sqrt(taps)
    return ws.astype(np.float32), wt.astype(np.float32)


def prep_inputs(cfg: Config, threads: int | None = None) -> dict:
    """Stacked raw features q, k, v [B, H, L, d] (float32 holding cfg.dtype
    values); the feature map consumes them token-major, i.e. transposed to
    [B, L, H, d]."""
    B, H = cfg.B, cfg.H
    out = {k: np.empty((B, H, cfg.L, cfg.d), np.float32) for k in ("q", "k", "v")}

    def one(bh):
        b, h = bh
        r = prep_head_inputs(cfg, b, h)
        for k in out:
            out[k][b, h] = r[k]

    n = threads or min(16, len(os.sched_getaffinity(0)))
    with _cf.ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        list(ex.map(one, [(b, h) for b in range(B) for h in range(H)]))
    return out


def grad_output(cfg: Config, branch: str = "s") -> np.ndarray:
    """Seeded gradient of a gated branch output, dOhat [B, L, H, d] ~ N(0, 1),
    rounded to cfg.dtype (the output layout of the branch); branch "s"
    (Softmax) or "l" (linear) draws an independent stream."""
    tid = {"s": "d_out", "l": "d_out_l"}[branch]
    out = np.empty((cfg.B, cfg.L, cfg.H, cfg.d), np.float32)
    for b in range(cfg.B):
        for h in range(cfg.H):
            out[b, :, h] = _store(cfg, _normal(cfg, tid, b, h, (cfg.L, cfg.d)))
    return out

