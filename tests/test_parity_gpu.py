"""GPU parity: every C-ABI entry point against the CPU fp64 oracle on the
same seeded inputs.  Tolerances (relative L2): fp32 storage 1e-4, bf16
storage 1e-2 on every branch output; fp32 states (P_fwd, P_rev, S_text)
1e-4 in both cases since the state arithmetic is fp32 throughout."""
import numpy as np
import pytest

from gpu_util import check_full as _check_full
from gpu_util import gpu_tensors, run_library
from vdn_inputs import CONFIGS, full_inputs

pytestmark = pytest.mark.gpu


# ---- the two small named configurations, in full ----
def test_tiny_fp32_full():
    _check_full(CONFIGS["tiny"])


def test_small_bf16_full():
    _check_full(CONFIGS["small"])


# ---- variants: paths, ragged tails, degenerate cases ----
VARIANTS = {
    # MFMA path with partial query and key tiles (N % 64 != 0, 5N % 128 != 0)
    "bf16_d64_ragged": CONFIGS["small"].replace(H=2, F=20, N=80, T=24),
    "bf16_d128_ragged": CONFIGS["small"].replace(H=2, d=128, F=15, N=112, T=40),
    # SIMT Softmax path for bf16 (N % 16 != 0, head dims 16 / 32)
    "bf16_d64_N37": CONFIGS["small"].replace(H=2, F=20, N=37, T=8),
    "bf16_d16": CONFIGS["small"].replace(H=3, d=16, F=20, N=48, T=8),
    "bf16_d32": CONFIGS["small"].replace(H=2, d=32, F=25, N=32, T=8),
    "f32_d128": CONFIGS["tiny"].replace(H=2, d=128, F=15, N=24, T=16),
    "f32_d64_B2": CONFIGS["tiny"].replace(B=2, H=2, d=64, F=20, N=20, T=5),
    # degenerate: short clips (all-dense Softmax, C = 1 and 2), no text
    "bf16_F5": CONFIGS["small"].replace(H=2, F=5, N=64, T=16),
    "bf16_F10": CONFIGS["small"].replace(H=2, F=10, N=64, T=16),
    "f32_F2_chunk1": CONFIGS["tiny"].replace(F=2, N=16, T=4),
    "bf16_T0": CONFIGS["small"].replace(H=2, F=20, N=64, T=0),
    "f32_T0": CONFIGS["tiny"].replace(T=0),
    # gates: zero write gate + unit decay; literal U(0,1) decay
    "bf16_beta0_alpha1": CONFIGS["small"].replace(H=2, F=20, N=64, beta="zero", alpha="unit"),
    "f32_alpha_u01": CONFIGS["tiny"].replace(alpha="u01"),
    "bf16_alpha_u01": CONFIGS["small"].replace(H=2, F=20, N=64, alpha="u01"),
    # no projections: out = Ohat_s + Ohat_l
    "bf16_noproj": CONFIGS["small"].replace(H=2, F=20, N=64, proj=False),
    "f32_noproj": CONFIGS["tiny"].replace(proj=False),
    # per-head gates, duplicated frames
    "bf16_headgates_dup": CONFIGS["small"].replace(H=2, F=40, N=64, gates="head", dup_frac=0.1),
}


@pytest.mark.parametrize("name", sorted(VARIANTS))
def test_variant(name):
    cfg = VARIANTS[name]
    if name == "f32_F2_chunk1":
        import softmax_attention_video_amd as vdn
        _check_full(cfg, vdn.Params(chunk_frames=1))
    else:
        _check_full(cfg)


@pytest.mark.parametrize("pk", [dict(anchors=0), dict(chunk_frames=3, window_chunks=2),
                                dict(chunk_frames=4, window_chunks=0),
                                dict(text_init_scale=1.0, rms_eps=1e-3, softmax_scale=0.2)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_params(pk, dtype):
    import softmax_attention_video_amd as vdn
    base = CONFIGS["tiny"] if dtype == "f32" else CONFIGS["small"].replace(H=2, N=64)
    cfg = base.replace(F=24 if pk.get("chunk_frames", 5) in (3, 4) else 20)
    _check_full(cfg, vdn.Params(**pk))


def test_deterministic():
    import torch
    cfg = CONFIGS["small"].replace(H=2, F=20, N=128, T=32)
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    a = run_library(cfg, t)
    b = run_library(cfg, t)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
    torch.cuda.synchronize()


def test_device_errors_raise():
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["small"].replace(H=1, F=20, N=64, T=8)
    t = gpu_tensors(cfg, full_inputs(cfg))
    with pytest.raises(vdn.VdnError) as e:
        vdn.window_softmax_fwd(t["q"], t["k"], t["v"], F=20, params=vdn.Params(chunk_frames=3))
    assert e.value.status == vdn.VDN_ERR_INVALID_ARG
    with pytest.raises(vdn.VdnError) as e:
        vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                     t["beta_text"], t["g_s"], t["g_l"], W_s=t["W_s"], W_l=None)
    assert e.value.status == vdn.VDN_ERR_INVALID_ARG
