"""Helpers shared by the GPU parity tests (no test functions here)."""
from __future__ import annotations

import sys

import numpy as np

DEV = "cuda:0"


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(cfg):
    import torch
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV).to(dtype)


def gpu_tensors(cfg, inp):
    """Upload the generator's (already rounded) arrays; bf16 casts are exact."""
    import torch
    dt = torch_dtype(cfg)
    t = {}
    for key in ("q", "k", "v", "k_text", "v_text"):
        t[key] = to_dev(inp[key], dt)
    for key in ("beta", "alpha", "beta_text", "g_s", "g_l", "gamma"):
        t[key] = to_dev(inp[key], torch.float32)
    t["W_s"] = to_dev(inp["W_s"], dt) if inp.get("W_s") is not None else None
    t["W_l"] = to_dev(inp["W_l"], dt) if inp.get("W_l") is not None else None
    return t


def to_np(x):
    return None if x is None else x.float().cpu().numpy().astype(np.float64)


def rel_l2(got, exp) -> float:
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    assert got.shape == exp.shape, (got.shape, exp.shape)
    assert np.isfinite(got).all(), "non-finite values in GPU output"
    den = np.linalg.norm(exp)
    return float(np.linalg.norm(got - exp) / (den if den > 0 else 1.0))


def run_library(cfg, t, params=None, with_parts=True):
    """Run every entry point once on the same inputs; returns numpy float64."""
    import torch
    import softmax_attention_video_amd as vdn
    B, H, L, d = t["q"].shape
    F = t["alpha"].shape[2]
    dt = torch_dtype(cfg)
    ohs = torch.empty((B, L, H, d), dtype=dt, device=DEV)
    ohl = torch.empty((B, L, H, d), dtype=dt, device=DEV)
    args = (t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
            t["beta_text"], t["g_s"], t["g_l"])
    out = vdn.attn_fwd(*args, gamma=t["gamma"], W_s=t["W_s"], W_l=t["W_l"], ohat_s=ohs,
                       ohat_l=ohl, params=params)
    res = {"out": out, "Ohat_s": ohs, "Ohat_l": ohl}
    if with_parts:
        sargs = (t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"], t["beta_text"])
        res["P_fwd"], res["S_text"] = vdn.scan_fwd(*sargs, params=params)
        res["P_rev"], _ = vdn.scan_rev(*sargs, params=params)
        res["sm"], res["lse"] = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], F, g_s=t["g_s"],
                                                       want_lse=True, params=params,
                                                       k_text=t["k_text"], v_text=t["v_text"])
    torch.cuda.synchronize()
    return {k: to_np(v) for k, v in res.items()}


def oracle_params(params):
    from oracle import vdn_oracle as O
    if params is None:
        return O.Params()
    return O.Params(chunk_frames=params.chunk_frames, window_chunks=params.window_chunks,
                    anchors=bool(params.anchors),
                    softmax_scale=params.softmax_scale if params.softmax_scale > 0 else None,
                    rms_eps=params.rms_eps, text_init_scale=params.text_init_scale,
                    text_softmax=bool(params.text_softmax))


def block_errors(got, exp, F):
    """Largest rel-L2 over the heads and over the (batch, head, frame) blocks
    of a [B, L, H, d] output."""
    got = np.asarray(got, np.float64)
    exp = np.asarray(exp, np.float64)
    B, L, H, d = exp.shape
    N = L // F
    g5 = got.reshape(B, F, N, H, d)
    e5 = exp.reshape(B, F, N, H, d)
    head = max(rel_l2(got[b, :, h], exp[b, :, h]) for b in range(B) for h in range(H))
    frame = max(rel_l2(g5[b, f, :, h], e5[b, f, :, h])
                for b in range(B) for h in range(H) for f in range(F))
    return head, frame


TOL = {"f32": 1e-4, "bf16": 1e-2}
TOL_STATE = 1e-4


def check_full(cfg, params=None, tol=None):
    """Every entry point on the full inputs of cfg against the oracle
    (vdn_attn over all heads); asserts the tolerances and returns the
    rel-L2 errors."""
    from oracle import vdn_oracle as O
    from vdn_inputs import full_inputs
    import softmax_attention_video_amd as vdn  # noqa: F401  (fails loudly if unbuilt)
    log(f"[parity] {cfg}")
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    got = run_library(cfg, t, params)
    op = oracle_params(params)
    ref = O.vdn_attn(inp, op)
    tol = tol or TOL[cfg.dtype]
    B, H, L, d = inp["q"].shape
    errs = {
        "P_fwd": rel_l2(got["P_fwd"], ref["P_fwd"]),
        "P_rev": rel_l2(got["P_rev"], ref["P_rev"]),
        "S_text": rel_l2(got["S_text"], ref["S_text"]) if cfg.T else float(np.abs(got["S_text"]).max()),
        "Ohat_s": rel_l2(got["Ohat_s"], ref["Ohat_s"].transpose(0, 2, 1, 3)),
        "Ohat_l": rel_l2(got["Ohat_l"], ref["Ohat_l"].transpose(0, 2, 1, 3)),
        "sm": rel_l2(got["sm"], ref["Ohat_s"].transpose(0, 2, 1, 3)),
        "lse": rel_l2(got["lse"], ref["lse"]),
        "out": rel_l2(got["out"].reshape(ref["out"].shape), ref["out"]),
    }
    # per head and per (head, frame) maxima beside the pooled figures, so
    # that one wrong head or frame cannot hide behind the others
    F = inp["alpha"].shape[2]
    for key, g_, r_ in (("Ohat_s", got["Ohat_s"], ref["Ohat_s"].transpose(0, 2, 1, 3)),
                        ("Ohat_l", got["Ohat_l"], ref["Ohat_l"].transpose(0, 2, 1, 3)),
                        ("sm", got["sm"], ref["Ohat_s"].transpose(0, 2, 1, 3))):
        errs[key + "_head_max"], errs[key + "_frame_max"] = block_errors(g_, r_, F)
    o_g = got["out"].reshape(ref["out"].shape)
    errs["out_frame_max"] = max(rel_l2(o_g[b, f * (L // F):(f + 1) * (L // F)],
                                       ref["out"][b, f * (L // F):(f + 1) * (L // F)])
                                for b in range(B) for f in range(F))
    log(f"[parity] rel-L2 {errs}")
    for key in ("P_fwd", "P_rev", "S_text"):
        assert errs[key] <= TOL_STATE, (key, errs)
    for key in ("Ohat_s", "Ohat_l", "sm", "out"):
        assert errs[key] <= tol, (key, errs)
    for key in ("Ohat_s", "Ohat_l", "sm"):
        assert errs[key + "_head_max"] <= tol, (key, errs)
        assert errs[key + "_frame_max"] <= tol, (key, errs)
    assert errs["out_frame_max"] <= tol, errs
    assert errs["lse"] <= 1e-5, errs
    return errs
