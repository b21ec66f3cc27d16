"""GPU parity of the Softmax-branch backward (vdn_window_softmax_bwd) against
the fp64 oracle: the GPU forward supplies the ungated output and the
log-sum-exp (as a training step would), the backward returns dq, dk, dv and
the gate gradient; the oracle differentiates its own forward.  SIMT and MFMA
paths, ragged tiles, no anchors, and sampled rows at full size."""
import numpy as np
import pytest

from gpu_util import DEV, TOL, gpu_tensors, log, oracle_params, rel_l2, to_np, to_dev
from oracle import softmax_bwd as SB
from vdn_inputs import CONFIGS, full_inputs, grad_output

pytestmark = pytest.mark.gpu


def _run(cfg, params=None):
    import torch
    import softmax_attention_video_amd as vdn
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    dout_np = grad_output(cfg)
    dout = to_dev(dout_np, t["q"].dtype)
    o, lse = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], cfg.F, want_lse=True, params=params)
    dq, dk, dv, dg = vdn.window_softmax_bwd(t["q"], t["k"], t["v"], o, lse, dout, cfg.F, g_s=t["g_s"],
                                            want_dg=True, params=params)
    torch.cuda.synchronize()
    return inp, dout_np, [to_np(x) for x in (dq, dk, dv, dg)]


def _check(cfg, params=None, tol=None):
    log(f"[bwd] {cfg}")
    inp, dout, got = _run(cfg, params)
    op = oracle_params(params)
    B, H, L, d = inp["q"].shape
    tol = tol or TOL[cfg.dtype]
    errs = {}
    for b in range(B):
        for h in range(H):
            sh = lambda x: x[b, h].astype(np.float64).reshape(cfg.F, cfg.N, -1)
            ref = SB.softmax_branch_bwd(sh(inp["q"]), sh(inp["k"]), sh(inp["v"]),
                                        inp["g_s"][b, h].reshape(cfg.F, cfg.N),
                                        dout[b, :, h].astype(np.float64).reshape(cfg.F, cfg.N, d), op)
            for name, g_, r in zip(("dq", "dk", "dv", "dg"), got, ref):
                e = rel_l2(g_[b, h], r.reshape(g_[b, h].shape))
                errs[name] = max(errs.get(name, 0.0), e)
    log(f"[bwd] max rel-L2 over heads {errs}")
    for name, e in errs.items():
        assert e <= tol, (name, errs)
    return errs


def test_bwd_tiny_fp32():
    _check(CONFIGS["tiny"])


def test_bwd_small_bf16():
    _check(CONFIGS["small"].replace(H=2))


VARIANTS = {
    "bf16_d128_ragged": CONFIGS["small"].replace(H=2, d=128, F=15, N=112, T=0),
    "bf16_d64_ragged": CONFIGS["small"].replace(H=2, F=20, N=80, T=0),
    "bf16_N37_simt": CONFIGS["small"].replace(H=2, F=20, N=37, T=0),
    "bf16_d32": CONFIGS["small"].replace(H=2, d=32, F=25, N=32, T=0),
    "f32_d128_B2": CONFIGS["tiny"].replace(B=2, H=2, d=128, F=15, N=24, T=0),
    "bf16_F5_dense": CONFIGS["small"].replace(H=2, F=5, N=64, T=0),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_bwd_variant(name):
    _check(VARIANTS[name])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_without_anchors(dtype):
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["tiny"] if dtype == "f32" else CONFIGS["small"].replace(H=2, F=20, N=64)
    _check(cfg, vdn.Params(anchors=0))


@pytest.mark.parametrize("name", ["medium", "h3"])
def test_bwd_full_size_sampled(name):
    """Full size, in the launch configuration the benchmark times: dq at
    sampled rows (anchor frames, chunk edges, random), dk and dv at sampled
    rows of one interior key frame, for two heads; and, over every row, the
    identity sum_k dV_k = sum_q g_s dOhat_q of each head."""
    import torch
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS[name]
    log(f"[bwd-large] {name}: generating inputs")
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    dout_np = grad_output(cfg)
    dout = to_dev(dout_np, t["q"].dtype)
    log(f"[bwd-large] {name}: forward + backward")
    o, lse = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], cfg.F, want_lse=True)
    dq, dk, dv, dg = vdn.window_softmax_bwd(t["q"], t["k"], t["v"], o, lse, dout, cfg.F, g_s=t["g_s"],
                                            want_dg=True)
    torch.cuda.synchronize()
    # identity over all rows, per head
    lhs = dv.float().sum(dim=2).double().cpu().numpy()                         # [B, H, d]
    gs = inp["g_s"].astype(np.float64)                                        # [B, H, L]
    rhs = np.einsum("bhl,blhd->bhd", gs, dout_np.astype(np.float64))
    e_sum = rel_l2(lhs, rhs)
    log(f"[bwd-large] {name}: sum_k dV vs sum_q dO rel-L2 {e_sum:.3e}")
    assert e_sum <= 1e-2
    N, F = cfg.N, cfg.F
    rng = np.random.default_rng(3)
    qrows = sorted({0, N - 1, (F - 1) * N, (F - 1) * N + 7, 5 * N, 5 * N - 1, (F // 2) * N + 3}
                   | set(int(x) for x in rng.choice(cfg.L, 16, replace=False)))
    qrows = np.array(qrows)
    kframe = F // 2 + 1
    krows = kframe * N + np.array([0, 1, N // 2, N - 1] + list(rng.choice(N, 8, replace=False)))
    for h in (0, cfg.H - 1):
        b = 0
        f64 = lambda x: x[b, h].astype(np.float64)
        log(f"[bwd-large] {name}: oracle rows, head {h}")
        rq, rk, rv = SB.softmax_bwd_rows(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["g_s"][b, h],
                                         dout_np[b, :, h].astype(np.float64), F, qrows, kframe, krows)
        gq = to_np(dq[b, h].index_select(0, torch.from_numpy(qrows).to(DEV)))
        gk = to_np(dk[b, h].index_select(0, torch.from_numpy(krows).to(DEV)))
        gv = to_np(dv[b, h].index_select(0, torch.from_numpy(krows).to(DEV)))
        errs = (rel_l2(gq, rq), rel_l2(gk, rk), rel_l2(gv, rv))
        log(f"[bwd-large] {name} h={h}: dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}")
        assert max(errs) <= TOL[cfg.dtype], errs
