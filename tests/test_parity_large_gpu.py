"""GPU parity at the full sizes of the medium, H3-scale and long-clip
configurations, in the launch configuration the benchmark times
(vdn_attn_fwd with default parameters, projections on).

The oracle cannot evaluate every row there, so it computes, one by one:
  - the chunk-boundary states P_fwd / P_rev and S_text of every head, in full;
  - Ohat_s, Ohat_l of every head at sampled token rows;
  - the projected output at sampled rows, which needs every head's
    Ohat_s / Ohat_l at those rows (all heads are evaluated at those rows).
Rows are sampled to cover anchor frames, chunk edges, the first and last
chunks, duplicated frames and random interior rows.
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

from gpu_util import DEV, gpu_tensors, log, rel_l2, to_np
from oracle import vdn_oracle as O
from vdn_inputs import CONFIGS, duplicated_frames, full_inputs

pytestmark = pytest.mark.gpu


def _rows(cfg, n_random=88, seed=0):
    N, F = cfg.N, cfg.F
    fr = [0, F - 1, 1, 4, 5, 9, 10, F // 2, F - 6, F - 5, F - 2]
    fr += duplicated_frames(cfg)[:3]
    rows = set()
    for f in fr:
        rows |= {f * N, f * N + N - 1, f * N + N // 2}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.choice(cfg.L, size=n_random, replace=False))
    return np.array(sorted(rows), np.int64)


def _head(cfg, inp, b, h, rows, want_softmax=True):
    return O.head_rows(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h], inp["beta"][b, h],
                       inp["alpha"][b, h], inp["k_text"][b, h], inp["v_text"][b, h],
                       inp["beta_text"][b, h], inp["g_s"][b, h], inp["g_l"][b, h], rows,
                       gamma=inp["gamma"], want_softmax=want_softmax)


@pytest.mark.parametrize("name", ["medium", "h3", "long"])
def test_full_size_sampled(name):
    import torch

    import softmax_attention_video_amd as vdn
    cfg = CONFIGS[name]
    log(f"[large] {name}: generating inputs {cfg}")
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    B, H, L, d = t["q"].shape
    dt = t["q"].dtype
    log(f"[large] {name}: vdn_attn_fwd")
    ohs = torch.empty((B, L, H, d), dtype=dt, device=DEV)
    ohl = torch.empty((B, L, H, d), dtype=dt, device=DEV)
    out = vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                       t["beta_text"], t["g_s"], t["g_l"], gamma=t["gamma"], W_s=t["W_s"],
                       W_l=t["W_l"], ohat_s=ohs, ohat_l=ohl)
    log(f"[large] {name}: vdn_attn_fwd with the MX-FP8 merge")
    out_mx = vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                          t["beta_text"], t["g_s"], t["g_l"], gamma=t["gamma"], W_s=t["W_s"],
                          W_l=t["W_l"], params=vdn.Params(merge_mxfp8=1))
    sargs = (t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"], t["beta_text"])
    P_f, S_t = vdn.scan_fwd(*sargs)
    P_r, _ = vdn.scan_rev(*sargs)
    torch.cuda.synchronize()
    rows = _rows(cfg)
    ridx = torch.from_numpy(rows).to(DEV)
    g_out = to_np(out[0].index_select(0, ridx))
    g_out_mx = to_np(out_mx[0].index_select(0, ridx))
    g_ohs = to_np(ohs[0].index_select(0, ridx))          # [R, H, d]
    g_ohl = to_np(ohl[0].index_select(0, ridx))
    heads_full = list(range(H))
    g_P = {h: (to_np(P_f[0, h]), to_np(P_r[0, h]), to_np(S_t[0, h])) for h in heads_full}
    del out, out_mx, ohs, ohl, P_f, P_r, S_t, t
    torch.cuda.empty_cache()

    log(f"[large] {name}: oracle on {len(rows)} rows x {H} heads")
    import threadpoolctl
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    ref = [None] * H
    # one BLAS thread per worker: heads run in parallel instead
    with threadpoolctl.threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {ex.submit(_head, cfg, inp, 0, h, rows): h for h in range(H)}
        for n_done, fut in enumerate(cf.as_completed(futs), 1):
            ref[futs[fut]] = fut.result()
            log(f"[large] {name}: oracle head {futs[fut]} done ({n_done}/{H})")
    errs = {}
    for h in heads_full:
        Pf, Pr, St = g_P[h]
        errs[f"P_fwd[h{h}]"] = rel_l2(Pf, ref[h]["P_fwd"])
        errs[f"P_rev[h{h}]"] = rel_l2(Pr, ref[h]["P_rev"])
        errs[f"S_text[h{h}]"] = rel_l2(St, ref[h]["S_text"])
    r_ohs = np.stack([ref[h]["Ohat_s"] for h in range(H)], axis=1)     # [R, H, d]
    r_ohl = np.stack([ref[h]["Ohat_l"] for h in range(H)], axis=1)
    errs["Ohat_s"] = rel_l2(g_ohs, r_ohs)
    errs["Ohat_l"] = rel_l2(g_ohl, r_ohl)
    # per head over the sampled rows: one wrong head cannot hide in the pool
    errs["Ohat_s_head_max"] = max(rel_l2(g_ohs[:, h], r_ohs[:, h]) for h in range(H))
    errs["Ohat_l_head_max"] = max(rel_l2(g_ohl[:, h], r_ohl[:, h]) for h in range(H))
    r_out = O.merge(r_ohs[None], r_ohl[None], inp["W_s"], inp["W_l"])[0]
    errs["out"] = rel_l2(g_out, r_out)
    # per-row check as well: no single sampled row may be far off
    row_err = np.linalg.norm(g_out - r_out, axis=1) / np.linalg.norm(r_out, axis=1)
    errs["out_row_max"] = float(row_err.max())
    # MX-FP8 merge: the oracle quantizes the branch outputs as the kernels
    # store them (bf16); codes near a rounding boundary may still differ, so
    # the bound is the one derived for this mode (5e-2)
    from oracle import mx_merge as MX
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()
    r_out_mx = MX.mx_merge(bf(r_ohs)[None], bf(r_ohl)[None], inp["W_s"], inp["W_l"])[0][0]
    errs["out_mx"] = rel_l2(g_out_mx, r_out_mx)
    log(f"[large] {name}: rel-L2 {errs}")
    assert errs["out_mx"] <= 5e-2, errs
    for key, v in errs.items():
        if key.startswith(("P_", "S_text")):
            assert v <= 1e-4, (key, errs)
    for key in ("Ohat_s", "Ohat_l", "out", "Ohat_s_head_max", "Ohat_l_head_max"):
        assert errs[key] <= 1e-2, (key, errs)
    assert errs["out_row_max"] <= 3e-2, errs
