"""GPU parity of the Softmax-branch backward with text keys
(params.text_softmax = 1: the T text tokens are keys of every query in the
same softmax) against the fp64 oracle, every gradient including dk_text and
dv_text: SIMT and MFMA paths, text counts below, at and off multiples of the
16-key groups, no anchors, two batches; and at the medium size whole-head
text gradients, sampled rows and the value-sum identity."""
import numpy as np
import pytest

from gpu_util import DEV, TOL, gpu_tensors, log, oracle_params, rel_l2, to_dev, to_np
from oracle import softmax_bwd as SB
from vdn_inputs import CONFIGS, full_inputs, grad_output

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dk_text", "dv_text")


def _run(cfg, params):
    import torch
    import softmax_attention_video_amd as vdn
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    dout_np = grad_output(cfg)
    dout = to_dev(dout_np, t["q"].dtype)
    o, lse = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], cfg.F, want_lse=True, params=params,
                                    k_text=t["k_text"], v_text=t["v_text"])
    got = vdn.window_softmax_bwd(t["q"], t["k"], t["v"], o, lse, dout, cfg.F, g_s=t["g_s"],
                                 want_dg=True, params=params, k_text=t["k_text"], v_text=t["v_text"])
    torch.cuda.synchronize()
    assert len(got) == 6
    return inp, dout_np, got


def _ref_head(cfg, inp, dout, op, b, h):
    sh = lambda x: x[b, h].astype(np.float64).reshape(cfg.F, cfg.N, -1)
    return SB.softmax_branch_bwd(sh(inp["q"]), sh(inp["k"]), sh(inp["v"]),
                                 inp["g_s"][b, h].reshape(cfg.F, cfg.N),
                                 dout[b, :, h].astype(np.float64).reshape(cfg.F, cfg.N, cfg.d), op,
                                 K_text=inp["k_text"][b, h].astype(np.float64),
                                 V_text=inp["v_text"][b, h].astype(np.float64))


def _check(cfg, params):
    log(f"[bwd-text] {cfg} {params}")
    inp, dout, got = _run(cfg, params)
    got = [to_np(x) for x in got]
    op = oracle_params(params)
    B, H = inp["q"].shape[:2]
    errs = {}
    for b in range(B):
        for h in range(H):
            ref = _ref_head(cfg, inp, dout, op, b, h)
            for name, g_, r in zip(NAMES, got, ref):
                assert np.isfinite(g_[b, h]).all(), name
                assert np.abs(r).max() > 0, f"reference {name} is zero: the case does not exercise it"
                errs[name] = max(errs.get(name, 0.0), rel_l2(g_[b, h], r.reshape(g_[b, h].shape)))
    log(f"[bwd-text] max rel-L2 over heads {errs}")
    bad = {k: e for k, e in errs.items() if not e <= TOL[cfg.dtype]}
    assert not bad, (bad, errs)


CASES = {
    "tiny_f32_simt": CONFIGS["tiny"],                                            # T = 8
    "bf16_d64_T37": CONFIGS["small"].replace(H=2, F=20, N=64, T=37),
    "bf16_d64_T16": CONFIGS["small"].replace(H=1, F=15, N=32, T=16),
    "bf16_d128_T5": CONFIGS["small"].replace(H=2, d=128, F=15, N=48, T=5),
    "bf16_d128_T200": CONFIGS["small"].replace(H=1, d=128, F=20, N=64, T=200),
    "bf16_N37_simt_T11": CONFIGS["small"].replace(H=2, F=20, N=37, T=11),
    "f32_d32_B2_T3": CONFIGS["tiny"].replace(B=2, H=2, d=32, F=15, N=24, T=3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bwd_text(name):
    import softmax_attention_video_amd as vdn
    _check(CASES[name], vdn.Params(text_softmax=1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_text_without_anchors(dtype):
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["tiny"] if dtype == "f32" else CONFIGS["small"].replace(H=2, F=20, N=64, T=21)
    _check(cfg, vdn.Params(text_softmax=1, anchors=0))


def test_bwd_text_medium():
    """Medium (B=1 H=16 d=128 F=100 N=384 T=512): head 0 in full against the
    oracle, dk_text and dv_text included; the last head at sampled dq rows;
    for every head sum_k dV_k + sum_t dV_text_t = sum_q g_s dOhat_q."""
    import torch
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["medium"]
    params = vdn.Params(text_softmax=1)
    inp, dout, got = _run(cfg, params)
    dq, dk, dv, dg, dkt, dvt = got
    lhs = (dv.float().sum(dim=2) + dvt.float().sum(dim=2)).double().cpu().numpy()
    rhs = np.einsum("bhl,blhd->bhd", inp["g_s"].astype(np.float64), dout.astype(np.float64))
    e_sum = rel_l2(lhs, rhs)
    log(f"[bwd-text] medium: value-sum identity rel-L2 {e_sum:.3e}")
    assert e_sum <= 1e-2
    op = oracle_params(params)
    log("[bwd-text] medium: oracle, head 0 in full")
    ref = _ref_head(cfg, inp, dout, op, 0, 0)
    errs = {n: rel_l2(to_np(x[0, 0]), r.reshape(x[0, 0].shape)) for n, x, r in zip(NAMES, got, ref)}
    log(f"[bwd-text] medium head 0: {errs}")
    assert max(errs.values()) <= TOL[cfg.dtype], errs
    h = cfg.H - 1
    rng = np.random.default_rng(7)
    qrows = np.array(sorted({0, cfg.N - 1, (cfg.F - 1) * cfg.N + 3}
                            | set(int(x) for x in rng.choice(cfg.L, 12, replace=False))))
    f64 = lambda x: x[0, h].astype(np.float64)
    rq, _, _ = SB.softmax_bwd_rows(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), inp["g_s"][0, h],
                                   dout[0, :, h].astype(np.float64), cfg.F, qrows, None, [], op,
                                   K_text=f64(inp["k_text"]), V_text=f64(inp["v_text"]))
    gq = to_np(dq[0, h].index_select(0, torch.from_numpy(qrows).to(DEV)))
    e = rel_l2(gq, rq)
    log(f"[bwd-text] medium head {h}: sampled dq rel-L2 {e:.3e}")
    assert e <= TOL[cfg.dtype]
