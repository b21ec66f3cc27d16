#!/usr/bin/env python3
"""Benchmark of the VDN attention forward on one MI355X.

One step = one vdn_attn_fwd call over the whole H3-scale layer (window/anchor
Softmax, the bidirectional VDA scan from the text state, the readout and the
gated merge through both output projections) with every input already
resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config h3]

The roofline object is for the dominant kernel (the window Softmax): its
algorithmic flops per launch divided by its mean launch time, measured with
HIP events that the library records around each launch on its own stream
inside the timed region.  cpu_baseline times the CPU fp64 oracle on a bounded
sample of the same workload and scales it to tokens/s.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (AMD spec: 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def flop_counts(cfg, pairs: int, chunk_frames: int = 5) -> dict:
    """Algorithmic flops of one forward as the library runs it (masked pairs
    not counted).  The scans: d = 64, 128 scan the frame maps directly
    (S <- T_f S + U_f, 2 d^3 per frame and direction); d = 16, 32 compose
    each chunk's maps (8 products of 2 d^3 per chunk and direction) and scan
    the chunks (2 d^3 per chunk and direction)."""
    B, H, d, F, N, L, T = cfg.B, cfg.H, cfg.d, cfg.F, cfg.N, cfg.L, cfg.T
    C = F // chunk_frames
    softmax = 4.0 * d * pairs * N * N * H * B
    scan = 2 * F * 2.0 * d ** 3 if d in (64, 128) else 2 * C * (16.0 + 2.0) * d ** 3
    vda = (6.0 * N * d * d * F          # A_f, W_f and the q.M readout
           + 4.0 * T * d * d            # A_text, W_text
           + 4.0 * d ** 3 * (F + 1)     # frame solves (+ text frame)
           + scan) * H * B              # both directions
    merge = 4.0 * B * L * (H * d) * cfg.D if cfg.proj else 0.0
    return {"softmax": softmax, "vda": vda, "merge": merge, "total": softmax + vda + merge}


def algorithmic_bytes(cfg) -> float:
    """Minimum HBM traffic of one forward (inputs read once, outputs written once)."""
    B, H, d, F, L, T, C = cfg.B, cfg.H, cfg.d, cfg.F, cfg.L, cfg.T, cfg.F // 5
    es = 2 if cfg.dtype == "bf16" else 4
    qkv = 3 * B * H * L * d * es
    gates = 3 * B * H * L * 4 + B * H * F * d * 4 + B * H * T * (2 * d * es + 4)
    states = 2 * B * H * (C + 1) * d * d * 4
    w = 2 * H * d * cfg.D * es
    out = B * L * cfg.D * es
    return float(qkv + gates + states + w + out)


def cpu_baseline(cfg, target_s: float = 30.0) -> dict:
    """The oracle, untouched, on a bounded sample: head (0, 0) in full for its
    chunk-boundary states plus S sampled query rows, and the merge for those
    rows; scaled to the whole layer in tokens/s."""
    import numpy as np
    import threadpoolctl

    from oracle import vdn_oracle as O
    from vdn_inputs import head_inputs

    h = head_inputs(cfg, 0, 0)
    rng = np.random.default_rng(7)
    S = 64
    t0 = time.perf_counter()
    while True:
        rows = np.sort(rng.choice(cfg.L, size=S, replace=False))
        t_a = time.perf_counter()
        O.head_rows(**h, rows=rows)
        t_head = time.perf_counter() - t_a
        if time.perf_counter() - t0 > target_s / 3 or S >= cfg.L:
            break
        S = min(cfg.L, S * 4)
    # split: the row-independent part (stats, solves, scans) vs per-row work
    t_a = time.perf_counter()
    O.head_rows(**h, rows=rows[:1], want_softmax=False)
    t_fixed = time.perf_counter() - t_a
    t_rows = max(t_head - t_fixed, 0.0)
    K = cfg.H * cfg.d
    xs = np.zeros((1, S, cfg.H, cfg.d))
    W = np.zeros((K, cfg.D))
    t_a = time.perf_counter()
    O.merge(xs, xs, W, W)
    t_merge = time.perf_counter() - t_a
    per_head = t_fixed + t_rows * cfg.L / S
    total = cfg.B * cfg.H * per_head + t_merge * cfg.B * cfg.L / S
    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    return {
        "value": cfg.B * cfg.L / total,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"head (b=0,h=0): full chunk-boundary scan ({t_fixed:.2f} s) + {S} random "
                   f"query rows ({t_rows:.2f} s); merge of {S} rows ({t_merge:.3f} s); scaled to "
                   f"{cfg.B * cfg.H} heads x {cfg.L} rows; wall {time.perf_counter() - t0:.1f} s"),
    }


COPY_KERNEL_TAG = "MulFunctor"      # torch.mul(x, 1, out=y): reads and writes its size once
SOFTMAX_KERNEL_TAG = "window_softmax_mfma_kernel<"   # the video-keys-only variant (", false>")


def traffic_from_counters(fetch_csv: str, write_csv: str, config: str, calib_bytes: int) -> dict:
    """HBM bytes per window-Softmax launch from two rocprofv3 --pmc CSVs.

    FETCH_SIZE / WRITE_SIZE are reported in KiB per dispatch.  Each is scaled
    by factor = known bytes / counter bytes of the calibration copy kernel
    (a torch elementwise copy of calib_bytes that reads and writes its size
    once), measured in the same run.
    """
    import csv
    import statistics

    def per_dispatch(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"]) * 1024.0
        return vals

    out = {}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        v = per_dispatch(path, counter)
        copies = [b for (k, _), b in v.items() if COPY_KERNEL_TAG in k]
        sm = [b for (k, _), b in v.items() if SOFTMAX_KERNEL_TAG in k and ", false>" in k]
        if not copies or not sm:
            raise SystemExit(f"{path}: calibration copy or softmax dispatches missing")
        factor = calib_bytes / statistics.median(copies)
        out[name] = {"counter_bytes_per_launch": statistics.median(sm), "copy_factor": factor,
                     "bytes_per_launch": statistics.median(sm) * factor, "launches": len(sm)}
    out["bytes_per_launch"] = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    out["config"] = config
    out["kernel_source_sha256"] = softmax_source_digest()
    return out


def softmax_source_digest() -> str:
    """Digest of the sources the window-Softmax kernel is compiled from; a
    stored traffic figure is only reported while it matches."""
    import hashlib
    h = hashlib.sha256()
    for f in ("k_window_softmax.hip", "window_items.h", "vdn_common.h", "vdn_internal.h"):
        with open(os.path.join(ROOT, "softmax_attention_video_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measure_prep(cfg, t, reps: int = 10, cpu: bool = True) -> dict:
    """VDA-Prep (vda_prep_fwd, the linear branch's feature map, upstream of the
    timed layer) on the layer's q, k, v laid out token-major: HIP-event time of
    one call, HBM-roofline figures, and the oracle on one head scaled to all."""
    import numpy as np
    import torch

    import softmax_attention_video_amd as vdn
    from vdn_inputs import GRIDS, prep_filters

    gh, gw = GRIDS[cfg.name]
    params = vdn.PrepParams(gh, gw)
    ws_np, wt_np = prep_filters(cfg)
    dev = t["q"].device
    src = [t[x].permute(0, 2, 1, 3).contiguous() for x in ("q", "k", "v")]
    wsd, wtd = torch.from_numpy(ws_np).to(dev), torch.from_numpy(wt_np).to(dev)
    outs = [torch.empty_like(t["q"]) for _ in range(3)]

    def run():
        vdn.prep_fwd(*src, wsd, wtd, cfg.F, params, *outs)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    B, H, L, d = t["q"].shape
    nbytes = 6 * B * L * H * d * t["q"].element_size() + ws_np.nbytes + wt_np.nbytes
    gbps = nbytes / (ms / 1e3) / 1e9
    res = {"entry": "vda_prep_fwd", "workload": f"{cfg.name}: B={B} H={H} d={d} F={cfg.F} grid={gh}x{gw}, "
                                                 "3x3 spatial x 5 centred temporal taps",
           "ms": ms, "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": gbps / PEAK_HBM_GBS, "algorithmic_bytes": nbytes}
    del src, outs
    if cpu:
        import threadpoolctl
        from oracle import vda_prep as OP
        from vdn_inputs import prep_head_inputs
        h = prep_head_inputs(cfg, 0, 0)
        op = OP.PrepParams(gh, gw)
        t0 = time.perf_counter()
        OP.prep_head(h["q"].astype(np.float64), h["k"].astype(np.float64), h["v"].astype(np.float64),
                     ws_np[0].astype(np.float64), wt_np[0].astype(np.float64), op)
        t_head = time.perf_counter() - t0
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
        res["cpu_baseline"] = {"value": B * L / (t_head * B * H), "unit": "tokens/s", "cores": int(threads),
                               "kind": "oracle", "sample": f"head (b=0,h=0) in full ({t_head:.2f} s), scaled to "
                                                           f"{B * H} heads"}
    return res


def measure_text(cfg, t, reps: int = 5) -> dict:
    """The same layer with the text keys inside the Softmax branch
    (params.text_softmax = 1: every video query also sees the T text keys):
    ms per vdn_attn_fwd call and the Softmax kernel's MFMA roofline figures,
    counting the extra F*N*T (query, text key) pairs."""
    import torch

    import softmax_attention_video_amd as vdn

    params = vdn.Params(text_softmax=1)
    B, H, L, d = t["q"].shape
    dev = t["q"].device
    dims = vdn.Dims(B, H, cfg.F, cfg.N, cfg.T, d, d, cfg.D)
    code = vdn.VDN_BF16 if t["q"].dtype == torch.bfloat16 else vdn.VDN_F32
    ws = torch.empty(vdn.workspace_bytes(dims, params, code), dtype=torch.uint8, device=dev)
    out = torch.empty((B, L, cfg.D), dtype=t["q"].dtype, device=dev)

    def run():
        vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                     t["beta_text"], t["g_s"], t["g_l"], gamma=t["gamma"], W_s=t["W_s"],
                     W_l=t["W_l"], out=out, workspace=ws, params=params)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    timer = vdn.KernelTimer(reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    k_ms = timer.read()
    timer.close()
    ms = e0.elapsed_time(e1) / reps
    pairs = int(vdn.window_plan(cfg.F)[0].sum())
    sm_flops = 4.0 * d * (pairs * cfg.N * cfg.N + cfg.F * cfg.N * cfg.T) * H * B
    ach = sm_flops / (float(k_ms.mean()) / 1e3) / 1e12
    del ws, out
    return {"entry": "vdn_attn_fwd with text_softmax = 1",
            "workload": f"{cfg.name} with its T={cfg.T} text keys visible to every video query",
            "ms_per_step": ms, "tokens_per_s": B * L / (ms / 1e3),
            "kernel": f"window_softmax_mfma_kernel<{d}, true>", "kernel_ms": float(k_ms.mean()),
            "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "softmax_flops": sm_flops}


def measure_bwd(cfg, t, reps: int = 3, text: bool = False) -> dict:
    """Backward of the Softmax branch (vdn_window_softmax_bwd) on the layer's
    q, k, v and gate, with a seeded random output gradient: the forward
    (g_s = NULL, with lse) supplies O_s and lse outside the timed region.
    HIP-event time of the call and of its two MFMA kernels (KernelTimer)."""
    import torch

    import softmax_attention_video_amd as vdn

    B, H, L, d = t["q"].shape
    dev = t["q"].device
    if t["q"].dtype != torch.bfloat16:
        return {}
    params = vdn.Params(text_softmax=1) if text else vdn.Params()
    kt_, vt_ = (t["k_text"], t["v_text"]) if text else (None, None)
    T = kt_.shape[2] if text else 0
    o, lse = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], cfg.F, want_lse=True, params=params,
                                    k_text=kt_, v_text=vt_)
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    dout = torch.randn((B, L, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    dims = vdn.Dims(B, H, cfg.F, cfg.N, T, d, d, H * d)
    p = params.c()
    ws = torch.empty(vdn.lib().vdn_softmax_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(p),
                                                              vdn.VDN_BF16), dtype=torch.uint8, device=dev)

    def run():
        return vdn.window_softmax_bwd(t["q"], t["k"], t["v"], o, lse, dout, cfg.F, g_s=t["g_s"],
                                      want_dg=True, workspace=ws, params=params, k_text=kt_,
                                      v_text=vt_)

    run()
    torch.cuda.synchronize()
    timer = vdn.KernelTimer(reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    k_ms = timer.read()
    timer.close()
    ms = e0.elapsed_time(e1) / reps
    pairs = int(vdn.window_plan(cfg.F)[0].sum())
    # S, dP, dV, dQ, dK: 5 products of 2 d per visible (query, key) pair; text keys are seen by every query
    flops = 10.0 * d * (pairs * cfg.N * cfg.N + cfg.L * T) * H * B
    ach = flops / (float(k_ms.mean()) / 1e3) / 1e12
    del ws, o, lse, dout
    if text:
        return {"entry": "vdn_window_softmax_bwd with text_softmax = 1 (also dk_text, dv_text)",
                "workload": f"{cfg.name}: Softmax branch backward with its T={T} text keys",
                "ms": ms, "kernel_ms": float(k_ms.mean()), "bound": "mfma", "achieved": ach,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                "algorithmic_flops": flops}
    return {"entry": "vdn_window_softmax_bwd (dq, dk, dv, dg_s)",
            "workload": f"{cfg.name}: Softmax branch backward, B={B} H={H} d={d} F={cfg.F} N={cfg.N}",
            "ms": ms, "kernel": f"softmax_bwd_dq_mfma_kernel<{d}, false> + softmax_bwd_dkdv_mfma_kernel<{d}>",
            "kernel_ms": float(k_ms.mean()), "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "algorithmic_flops": flops,
            "executed_mfma_flops": 1.4 * flops,
            "note": "S and dP are computed in both kernels: 14 d MFMA flops per pair against the 10 d counted"}


def measure_merge_bwd(cfg, t, reps: int = 3) -> dict:
    """Backward of the merge (vdn_merge_bwd) at the layer's shape with seeded
    random branch outputs and output gradient: HIP-event time of the call
    (four GEMMs and the three token-contiguous transposes dW needs)."""
    import torch

    import softmax_attention_video_amd as vdn

    B, H, L, d = t["q"].shape
    dev = t["q"].device
    D = t["W_s"].shape[1]
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    r = lambda *s_: torch.randn(*s_, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    os_, ol_, dout = r(B, L, H, d), r(B, L, H, d), r(B, L, D)
    dims = vdn.Dims(B, H, cfg.F, cfg.N, 0, d, d, D)
    p = vdn.Params().c()
    ws = torch.empty(vdn.lib().vdn_merge_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(p), vdn.VDN_BF16),
                     dtype=torch.uint8, device=dev)

    def run():
        return vdn.merge_bwd(dout, os_, ol_, t["W_s"], t["W_l"], cfg.F, workspace=ws)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 4 * 2.0 * B * L * (H * d) * D
    ach = flops / (ms / 1e3) / 1e12
    del ws, os_, ol_, dout
    return {"entry": "vdn_merge_bwd (d_ohat_s, d_ohat_l, dW_s, dW_l)",
            "workload": f"{cfg.name} merge backward: M={B * L} tokens, K={H * d}, D={D}",
            "ms": ms, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "algorithmic_flops": flops,
            "note": "time of the whole call, the three transposes for dW included"}


def measure_vda_bwd(cfg, t, reps: int = 5, cpu: bool = True) -> dict:
    """Backward of the linear branch (vda_bwd) on the layer's inputs with a
    seeded random gradient of Ohat_l: HIP-event time of the whole call and,
    through the library's kernel timer, of its longest kernel, the readout
    adjoint (recompute q M, RMSNorm/gate adjoint, dq = dO M^T, G = Q^T dO).
    That kernel is bound by HBM (6 N d^2 flops per frame against the bytes
    of q, dOhat, dq and G): its algorithmic bytes per launch are q and
    dOhat read once, dq written once (2 B each per element), G written (fp32
    d x d per frame) and the chunk-boundary states read once (fp32)."""
    import torch

    import softmax_attention_video_amd as vdn

    B, H, L, d = t["q"].shape
    dev = t["q"].device
    if t["q"].dtype != torch.bfloat16:
        return {}
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    dout = torch.randn((B, L, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    dims = vdn.Dims(B, H, cfg.F, cfg.N, cfg.T, d, d, H * d)
    p = vdn.Params().c()
    ws = torch.empty(vdn.lib().vda_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(p), vdn.VDN_BF16),
                     dtype=torch.uint8, device=dev)

    def run():
        return vdn.vda_bwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                           t["beta_text"], t["g_l"], dout, gamma=t["gamma"], want_dg=True,
                           want_dgamma=True, workspace=ws)

    run()
    torch.cuda.synchronize()
    timer = vdn.KernelTimer(reps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    k_ms = timer.read()
    timer.close()
    ms = e0.elapsed_time(e1) / reps
    C = cfg.F // 5
    nbytes = 3.0 * B * H * L * d * 2 + B * H * cfg.F * d * d * 4 + 2.0 * B * H * (C + 1) * d * d * 4
    flops = 6.0 * B * H * L * d * d
    kms = float(k_ms.mean())
    gbps = nbytes / (kms / 1e3) / 1e9
    cpu_res = None
    if cpu:
        # the oracle on head (0, 0) of the same inputs, in full, scaled to all heads
        import numpy as np
        import threadpoolctl
        from oracle import vda_bwd as VB
        f64 = lambda x: x.detach().float().cpu().numpy().astype(np.float64)
        hd = {key: f64(t[key][0, 0]) for key in ("q", "k", "v", "beta", "alpha", "k_text", "v_text",
                                                 "beta_text", "g_l")}
        t0 = time.perf_counter()
        VB.linear_branch_bwd(hd["q"], hd["k"], hd["v"], hd["beta"], hd["alpha"], hd["k_text"], hd["v_text"],
                             hd["beta_text"], hd["g_l"], f64(t["gamma"]), f64(dout[0, :, 0]))
        t_head = time.perf_counter() - t0
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
        cpu_res = {"value": B * L / (t_head * B * H), "unit": "tokens/s", "cores": int(threads),
                   "kind": "oracle",
                   "sample": f"head (b=0,h=0) in full ({t_head:.2f} s), scaled to {B * H} heads"}
    del ws, dout
    return {"entry": "vda_bwd (dq, dk, dv, dbeta, dalpha, text gradients, dg_l, dgamma)",
            "workload": f"{cfg.name}: linear-branch backward, B={B} H={H} d={d} F={cfg.F} N={cfg.N} T={cfg.T}",
            "ms": ms, "tokens_per_s": B * L / (ms / 1e3),
            "kernel": f"vda_bwd_readout_mfma_kernel<{d}>", "kernel_ms": kms, "bound": "hbm",
            "achieved": gbps, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBS,
            "algorithmic_bytes": nbytes, "kernel_flops": flops,
            "kernel_tflops": flops / (kms / 1e3) / 1e12, "cpu_baseline": cpu_res}


PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 / MX-FP8 MFMA (2 x the bf16 peak)


def measure_mx(cfg, t, reps: int = 10) -> dict:
    """The merge (vdn_merge_fwd) on the layer's branch outputs, bf16 against
    MX-FP8 (params.merge_mxfp8 = 1: quantization of both operands included),
    and the layer step with the MX-FP8 merge.  HIP-event times on the stream."""
    import torch

    import softmax_attention_video_amd as vdn

    B, H, L, d = t["q"].shape
    dev = t["q"].device
    if t["W_s"] is None or t["q"].dtype != torch.bfloat16:
        return {}
    ohs = torch.empty((B, L, H, d), dtype=t["q"].dtype, device=dev)
    ohl = torch.empty_like(ohs)
    mx = vdn.Params(merge_mxfp8=1)
    dims = vdn.Dims(B, H, cfg.F, cfg.N, cfg.T, d, d, cfg.D)
    ws = torch.empty(vdn.workspace_bytes(dims, mx, vdn.VDN_BF16), dtype=torch.uint8, device=dev)
    out = torch.empty((B, L, cfg.D), dtype=t["q"].dtype, device=dev)

    def layer(params):
        vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                     t["beta_text"], t["g_s"], t["g_l"], gamma=t["gamma"], W_s=t["W_s"],
                     W_l=t["W_l"], out=out, ohat_s=ohs, ohat_l=ohl, workspace=ws, params=params)

    def merge(params):
        vdn.merge_fwd(ohs, ohl, t["W_s"], t["W_l"], cfg.F, params=params, out=out, workspace=ws)

    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    ms_layer = timed(lambda: layer(mx), 5)
    ms_bf16 = timed(lambda: merge(None), reps)
    ms_mx = timed(lambda: merge(mx), reps)
    flops = 4.0 * B * L * (H * d) * cfg.D
    del ws, out, ohs, ohl
    return {"entry": "vdn_merge_fwd (bf16 vs merge_mxfp8 = 1); vdn_attn_fwd with merge_mxfp8 = 1",
            "workload": f"{cfg.name} merge: M={B * L} tokens, K=2x{H * d}, D={cfg.D}",
            "merge_bf16_ms": ms_bf16, "merge_mx_ms": ms_mx,
            "bound": "mfma", "achieved": flops / (ms_mx / 1e3) / 1e12, "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": flops / (ms_mx / 1e3) / 1e12 / PEAK_FP8_TFLOPS,
            "bf16_achieved": flops / (ms_bf16 / 1e3) / 1e12, "bf16_frac":
            flops / (ms_bf16 / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
            "layer_ms_per_step": ms_layer, "layer_tokens_per_s": B * L / (ms_layer / 1e3),
            "note": "reduced precision (MX-FP8 operands); not the headline"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="h3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prep", action="store_true",
                    help="skip the separate VDA-Prep (vda_prep_fwd) measurement")
    ap.add_argument("--no-text", action="store_true",
                    help="skip the separate text-keys-in-Softmax measurement")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the separate MX-FP8 merge measurement")
    ap.add_argument("--no-vda-bwd", action="store_true",
                    help="skip the linear-branch backward leg")
    ap.add_argument("--no-bwd", action="store_true",
                    help="skip the separate Softmax-backward measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one elementwise copy of this many MiB before timing "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 counter CSVs into the traffic JSON and exit")
    args = ap.parse_args()
    if args.traffic_from:
        res = traffic_from_counters(*args.traffic_from, config=args.config,
                                    calib_bytes=(args.calib_copy_mib or 1024) << 20)
        path = os.path.join(ROOT, "profiles", f"window_softmax_{args.config}_traffic.json")
        with open(path, "w") as fh:
            json.dump(res, fh, indent=1)
        print(json.dumps(res))
        return 0
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); the "
              "multi-GPU (head-sharded) path is not built.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import softmax_attention_video_amd as vdn
    from vdn_inputs import CONFIGS, full_inputs

    cfg = CONFIGS[args.config]
    dev = "cuda:0"
    t_gen = time.perf_counter()
    inp = full_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    f32 = torch.float32
    t = {}
    for key in ("q", "k", "v", "k_text", "v_text"):
        t[key] = torch.from_numpy(inp.pop(key)).to(dev).to(dt)
    for key in ("beta", "alpha", "beta_text", "g_s", "g_l", "gamma"):
        t[key] = torch.from_numpy(inp.pop(key)).to(dev)
    W_s, W_l = inp.pop("W_s"), inp.pop("W_l")
    t["W_s"] = torch.from_numpy(W_s).to(dev).to(dt) if W_s is not None else None
    t["W_l"] = torch.from_numpy(W_l).to(dev).to(dt) if W_l is not None else None
    del inp, W_s, W_l
    print(f"[bench] inputs for {cfg.name} ready in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    B, H, L, d = t["q"].shape
    dims = vdn.Dims(B, H, cfg.F, cfg.N, cfg.T, d, d, cfg.D)
    ws = torch.empty(vdn.workspace_bytes(dims, None, vdn.VDN_BF16 if dt == torch.bfloat16
                                         else vdn.VDN_F32), dtype=torch.uint8, device=dev)
    out = torch.empty((B, L, cfg.D), dtype=dt, device=dev)

    def step():
        vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                     t["beta_text"], t["g_s"], t["g_l"], gamma=t["gamma"], W_s=t["W_s"],
                     W_l=t["W_l"], out=out, workspace=ws)

    if args.calib_copy_mib:
        n = (args.calib_copy_mib << 20) // 4
        xa = torch.ones(n, dtype=torch.float32, device=dev)
        xb = torch.empty_like(xa)
        torch.mul(xa, 1.0, out=xb)
        torch.cuda.synchronize()
        del xa, xb
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = vdn.KernelTimer(args.steps)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    k_ms = timer.read()
    timer.close()
    ms_step = ms_total / args.steps
    print(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step; window Softmax kernel "
          f"{k_ms.mean():.3f} ms (min {k_ms.min():.3f}, max {k_ms.max():.3f})",
          file=sys.stderr, flush=True)

    pairs = int(vdn.window_plan(cfg.F)[0].sum())     # visible (query, key) frame pairs
    fl = flop_counts(cfg, pairs)
    tok_s = B * L / (ms_step / 1e3)
    tflops = fl["total"] / (ms_step / 1e3) / 1e12
    k_tflops = fl["softmax"] / (k_ms.mean() / 1e3) / 1e12

    traffic = None
    prof = os.path.join(ROOT, "profiles", f"window_softmax_{cfg.name}_traffic.json")
    if os.path.exists(prof):
        with open(prof) as fh:
            rec = json.load(fh)
        if rec.get("kernel_source_sha256") == softmax_source_digest():
            traffic = rec.get("bytes_per_launch")

    res = {
        "metric": "VDN attention fwd video tokens/s (1 GPU)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of the named configuration)",
        "config": {"workload": f"{cfg.name}: VDN attention layer B={B} H={H} d={d} F={cfg.F} "
                               f"N={cfg.N} T={cfg.T} D={cfg.D}",
                   "B": B, "H": H, "d": d, "F": cfg.F, "N": cfg.N, "T": cfg.T, "D": cfg.D,
                   "visible_frame_pairs": pairs},
        "tflops": tflops,
        "pct_bf16_mfma_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "flops_per_step": fl,
        "roofline": {
            "kernel": f"window_softmax_mfma_kernel<{d}, false>",
            "bound": "mfma",
            "achieved": k_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": k_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "kernel_ms": float(k_ms.mean()),
        },
    }
    if not args.no_prep:
        from vdn_inputs import GRIDS
        if cfg.name in GRIDS:
            res["vda_prep"] = measure_prep(cfg, t, cpu=not args.no_cpu_baseline)
            print(f"[bench] vda_prep_fwd: {res['vda_prep']['ms']:.3f} ms, "
                  f"{res['vda_prep']['achieved']:.0f} GB/s", file=sys.stderr, flush=True)
    if not args.no_text and cfg.T > 0 and cfg.dtype == "bf16":
        res["text_softmax"] = measure_text(cfg, t)
        print(f"[bench] text keys in the Softmax: {res['text_softmax']['ms_per_step']:.3f} ms/step, "
              f"Softmax kernel {res['text_softmax']['kernel_ms']:.3f} ms", file=sys.stderr, flush=True)
    if not args.no_mx and cfg.proj and cfg.dtype == "bf16":
        res["merge_mxfp8"] = measure_mx(cfg, t)
        r = res["merge_mxfp8"]
        print(f"[bench] merge: bf16 {r['merge_bf16_ms']:.3f} ms, MX-FP8 {r['merge_mx_ms']:.3f} ms; "
              f"layer with the MX-FP8 merge {r['layer_ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)
    if not args.no_bwd and cfg.dtype == "bf16":
        res["softmax_bwd"] = measure_bwd(cfg, t)
        r = res["softmax_bwd"]
        print(f"[bench] Softmax backward: {r['ms']:.3f} ms, kernels {r['kernel_ms']:.3f} ms, "
              f"{r['achieved']:.0f} TFLOP/s", file=sys.stderr, flush=True)
        if "text_softmax" in res:
            res["text_softmax"]["bwd"] = r = measure_bwd(cfg, t, text=True)
            print(f"[bench] Softmax backward with text keys: {r['ms']:.3f} ms, kernels {r['kernel_ms']:.3f} ms, "
                  f"{r['achieved']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_bwd and cfg.proj and cfg.dtype == "bf16" and (cfg.B * cfg.L) % 128 == 0:
        res["merge_bwd"] = r = measure_merge_bwd(cfg, t)
        print(f"[bench] merge backward: {r['ms']:.3f} ms, {r['achieved']:.0f} TFLOP/s", file=sys.stderr,
              flush=True)
    if not args.no_vda_bwd and cfg.dtype == "bf16":
        res["vda_bwd"] = measure_vda_bwd(cfg, t, cpu=not args.no_cpu_baseline)
        r = res["vda_bwd"]
        print(f"[bench] linear-branch backward: {r['ms']:.3f} ms, readout adjoint {r['kernel_ms']:.3f} ms, "
              f"{r['achieved']:.0f} GB/s", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
