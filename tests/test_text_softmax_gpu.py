"""GPU parity of the text-aware Softmax option (params.text_softmax = 1: the
T text keys join every video query's softmax, anchors included) against the
fp64 oracle.  Whole-operator checks (vdn_attn_fwd and every standalone entry
point) on the SIMT and MFMA paths, ragged text lengths around the 16-key
groups and the 96 / 128-key tiles, and sampled rows at the medium and
H3-scale sizes through vdn_window_softmax_fwd."""
import numpy as np
import pytest

from gpu_util import DEV, TOL, check_full, gpu_tensors, log, rel_l2, to_np
from oracle import vdn_oracle as O
from vdn_inputs import CONFIGS, full_inputs

pytestmark = pytest.mark.gpu

SMALL = CONFIGS["small"]
CASES = {
    "tiny_f32": CONFIGS["tiny"],                                        # SIMT fp32, T = 8
    "small_bf16": SMALL,                                                # MFMA d = 64, T = 64
    # MFMA d = 128 (96-key tiles): one ragged 16-key group at the text end
    "bf16_d128_T77": SMALL.replace(H=2, d=128, F=15, N=112, T=77),
    "bf16_d128_T192": SMALL.replace(H=2, d=128, F=15, N=64, T=192),     # two whole tiles
    "bf16_d128_T1": SMALL.replace(H=2, d=128, F=20, N=48, T=1),
    # MFMA d = 64 (128-key tiles)
    "bf16_d64_T5": SMALL.replace(H=2, F=20, N=80, T=5),
    "bf16_d64_T130": SMALL.replace(H=2, F=20, N=32, T=130),
    "bf16_d64_T0": SMALL.replace(H=2, F=20, N=64, T=0),
    # SIMT paths: bf16 with N % 16 != 0, fp32 with B = 2
    "bf16_N37_T10": SMALL.replace(H=2, F=20, N=37, T=10),
    "f32_d64_B2_T5": CONFIGS["tiny"].replace(B=2, H=2, d=64, F=20, N=20, T=5),
    # short clip: every frame dense, text on top
    "bf16_F5_T24": SMALL.replace(H=2, F=5, N=64, T=24),
}


@pytest.mark.parametrize("name", list(CASES))
def test_text_softmax_full(name):
    import softmax_attention_video_amd as vdn
    check_full(CASES[name], vdn.Params(text_softmax=1))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_text_softmax_without_anchors(dtype):
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["tiny"] if dtype == "f32" else SMALL.replace(H=2, F=20, N=64, T=40)
    check_full(cfg, vdn.Params(text_softmax=1, anchors=0))


def test_text_softmax_off_ignores_text():
    """With the option off, text pointers given to the Softmax entry point
    change nothing (bit-identical to the call without them)."""
    import torch
    import softmax_attention_video_amd as vdn
    cfg = SMALL.replace(H=2, F=20, N=64, T=40)
    t = gpu_tensors(cfg, full_inputs(cfg))
    a, la = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], cfg.F, g_s=t["g_s"], want_lse=True)
    b, lb = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], cfg.F, g_s=t["g_s"], want_lse=True,
                                   k_text=t["k_text"], v_text=t["v_text"])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def _rows(cfg, n_random=32, seed=1):
    N, F = cfg.N, cfg.F
    rows = set()
    for f in (0, F - 1, 1, 4, 5, F // 2, F - 2):
        rows |= {f * N, f * N + N - 1, f * N + N // 2}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.choice(cfg.L, size=n_random, replace=False))
    return np.array(sorted(rows), np.int64)


@pytest.mark.parametrize("name", ["medium", "h3"])
def test_text_softmax_full_size_sampled(name):
    import torch
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS[name]
    log(f"[text-large] {name}: generating inputs {cfg}")
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    log(f"[text-large] {name}: vdn_window_softmax_fwd with {cfg.T} text keys")
    params = vdn.Params(text_softmax=1)
    out, lse = vdn.window_softmax_fwd(t["q"], t["k"], t["v"], cfg.F, g_s=t["g_s"], want_lse=True,
                                      params=params, k_text=t["k_text"], v_text=t["v_text"])
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    rows = _rows(cfg)
    rt = torch.from_numpy(rows).to(DEV)
    op = O.Params(text_softmax=True)
    N, d = cfg.N, cfg.d
    for h in (0, cfg.H - 1):
        Kf = inp["k"][0, h].astype(np.float64).reshape(cfg.F, N, d)
        Vf = inp["v"][0, h].astype(np.float64).reshape(cfg.F, N, d)
        exp_o = np.zeros((len(rows), d))
        exp_l = np.zeros(len(rows))
        for f in np.unique(rows // N):
            sel = np.nonzero(rows // N == f)[0]
            o, l = O.softmax_rows(inp["q"][0, h][rows[sel]], int(f), Kf, Vf, op,
                                  inp["k_text"][0, h], inp["v_text"][0, h])
            exp_o[sel] = inp["g_s"][0, h][rows[sel]][:, None] * o
            exp_l[sel] = l
        got_o = to_np(out[0, :, h].index_select(0, rt))
        got_l = to_np(lse[0, h].index_select(0, rt))
        eo, el = rel_l2(got_o, exp_o), rel_l2(got_l, exp_l)
        log(f"[text-large] {name} h={h}: Ohat_s rel-L2 {eo:.3e}, lse rel-L2 {el:.3e}")
        assert eo <= TOL[cfg.dtype] and el <= 1e-5
