"""GPU parity of the MX-FP8 merge (vdn_params.merge_mxfp8) against the fp64
oracle: the quantizer bit for bit (codes and scale bytes) on seeded bf16
inputs with zero, tiny, tie and saturating blocks; the merge alone on the
same bf16 operands (identical codes, so only fp32 accumulation and the bf16
output differ); and the whole operator, whose branch outputs are quantized
as the kernels store them."""
import numpy as np
import pytest

from gpu_util import DEV, check_full, gpu_tensors, log, rel_l2, to_np
from oracle import mx_merge as MX
from oracle import vdn_oracle as O
from vdn_inputs import CONFIGS, full_inputs

pytestmark = pytest.mark.gpu

TOL_MX_END_TO_END = 5e-2


def _bf16(a):
    """Round to bf16 (the storage type); returns the float64 values and the device tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy(), t.to(DEV)


def _quant_inputs(rows, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, 256)) * np.exp2(rng.integers(-30, 30, (rows, 1)))
    x[0] = 0.0                                           # zero blocks
    x[1, :32] = 2.0 ** -133                              # smallest bf16 subnormals
    x[1, 32:64] = -(2.0 ** -130)
    pos = MX.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2                      # ties in scale units (5 significant bits)
    for r in range(2, 6):                                # blocks of exact ties, scale 2^(r - 4)
        blk = np.resize(mids, 256)
        blk[::32] = 256.0                                # each block's max sets the scale
        x[r] = blk * 2.0 ** (r - 4) * np.where(np.arange(256) % 3 == 0, -1, 1)
    x[6] = np.resize([500.0, 470.0, 448.0, 300.0], 256)  # saturation (scale 1)
    x[7, :] = -0.0
    return x


@pytest.mark.parametrize("rows", [8, 1000])
def test_quantize_bit_exact(rows):
    import torch
    import softmax_attention_video_amd as vdn
    xv, xd = _bf16(_quant_inputs(rows, rows))
    codes, scales = vdn.mx_quantize(xd)
    torch.cuda.synchronize()
    want_c, want_s = MX.mx_quantize(xv)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:5].tolist()}: " \
                          f"{got_c[tuple(bad[0])]:#x} vs {want_c[tuple(bad[0])]:#x} for {xv[tuple(bad[0])]!r}"
    np.testing.assert_array_equal(got_s, want_s)


def _merge_case(B, L, H, d, D, seed):
    rng = np.random.default_rng(seed)
    os_v, os_d = _bf16(rng.standard_normal((B, L, H, d)) * rng.choice([1e-3, 1.0, 30.0], (B, L, H, 1)))
    ol_v, ol_d = _bf16(rng.standard_normal((B, L, H, d)))
    ws_v, ws_d = _bf16(rng.standard_normal((H * d, D)) / np.sqrt(H * d))
    wl_v, wl_d = _bf16(rng.standard_normal((H * d, D)) / np.sqrt(H * d))
    return (os_v, ol_v, ws_v, wl_v), (os_d, ol_d, ws_d, wl_d)


# (B, L, H, d, D, F): ragged row and column tiles; two batches; the H3 widths
@pytest.mark.parametrize("B,L,H,d,D,F", [(1, 600, 4, 64, 200, 120), (2, 250, 2, 32, 256, 50),
                                         (1, 1000, 24, 128, 3072, 100)])
def test_merge_fwd_mx_parity(B, L, H, d, D, F):
    import torch
    import softmax_attention_video_amd as vdn
    ref_in, dev_in = _merge_case(B, L, H, d, D, seed=L + D)
    log(f"[mx] merge B={B} L={L} H={H} d={d} D={D}")
    got = vdn.merge_fwd(*dev_in, F=F, params=vdn.Params(merge_mxfp8=1))
    ref = vdn.merge_fwd(*dev_in, F=F)          # the bf16 merge
    torch.cuda.synchronize()
    want_mx, _ = MX.mx_merge(*ref_in)
    want = O.merge(*ref_in)
    e_mx, e_bf = rel_l2(to_np(got), want_mx), rel_l2(to_np(ref), want)
    e_q = rel_l2(want_mx, want)
    # per output row as well (the last, partial row and column tiles included):
    # no row may hide in the pooled figure
    g_bf = to_np(ref).reshape(-1, D)
    w_bf = np.asarray(want).reshape(-1, D)
    row_bf = np.linalg.norm(g_bf - w_bf, axis=1) / np.maximum(np.linalg.norm(w_bf, axis=1), 1e-30)
    log(f"[mx] rel-L2 MX vs MX oracle {e_mx:.3e}, bf16 vs exact {e_bf:.3e} (MX vs exact {e_q:.3e}), "
        f"bf16 row max {row_bf.max():.3e}")
    assert e_mx <= 1e-2 and e_bf <= 1e-2
    assert row_bf.max() <= 3e-2, row_bf.max()


@pytest.mark.parametrize("name", ["small", "ragged"])
def test_attn_fwd_mx_end_to_end(name):
    import torch
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["small"] if name == "small" else CONFIGS["small"].replace(H=2, d=128, F=15, N=112, T=40)
    inp = full_inputs(cfg)
    t = gpu_tensors(cfg, inp)
    log(f"[mx] vdn_attn_fwd with the MX-FP8 merge: {cfg}")
    params = vdn.Params(merge_mxfp8=1)
    B, H, L, d = t["q"].shape
    ohs = torch.empty((B, L, H, d), dtype=t["q"].dtype, device=DEV)
    ohl = torch.empty_like(ohs)
    out = vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                       t["beta_text"], t["g_s"], t["g_l"], gamma=t["gamma"], W_s=t["W_s"],
                       W_l=t["W_l"], ohat_s=ohs, ohat_l=ohl, params=params)
    torch.cuda.synchronize()
    ref = O.vdn_attn(inp)
    r_ohs = ref["Ohat_s"].transpose(0, 2, 1, 3)
    r_ohl = ref["Ohat_l"].transpose(0, 2, 1, 3)
    # the branch outputs themselves are unchanged by the merge mode
    assert rel_l2(to_np(ohs), r_ohs) <= 1e-2 and rel_l2(to_np(ohl), r_ohl) <= 1e-2
    bf = lambda x: _bf16(x)[0]
    want, _ = MX.mx_merge(bf(r_ohs), bf(r_ohl), inp["W_s"], inp["W_l"])
    err = rel_l2(to_np(out), want)
    log(f"[mx] end-to-end rel-L2 {err:.3e}")
    assert err <= TOL_MX_END_TO_END


def test_mx_rejected_where_unsupported():
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["tiny"]                       # fp32 storage
    t = gpu_tensors(cfg, full_inputs(cfg))
    with pytest.raises(vdn.VdnError) as e:
        vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                     t["beta_text"], t["g_s"], t["g_l"], W_s=t["W_s"], W_l=t["W_l"],
                     params=vdn.Params(merge_mxfp8=1))
    assert e.value.status == vdn.VDN_ERR_UNSUPPORTED
    cfg = CONFIGS["small"].replace(H=2, F=20, N=64, proj=False)
    t = gpu_tensors(cfg, full_inputs(cfg))
    with pytest.raises(vdn.VdnError) as e:
        vdn.attn_fwd(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"],
                     t["beta_text"], t["g_s"], t["g_l"], params=vdn.Params(merge_mxfp8=1))
    assert e.value.status == vdn.VDN_ERR_INVALID_ARG


def test_mx_mode_leaves_default_path_unchanged():
    """The default merge is bit-identical before and after an MX-FP8 call."""
    import torch
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["small"].replace(H=2, F=20, N=64, T=16)
    t = gpu_tensors(cfg, full_inputs(cfg))
    args = (t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["k_text"], t["v_text"], t["beta_text"],
            t["g_s"], t["g_l"])
    a = vdn.attn_fwd(*args, gamma=t["gamma"], W_s=t["W_s"], W_l=t["W_l"]).clone()
    vdn.attn_fwd(*args, gamma=t["gamma"], W_s=t["W_s"], W_l=t["W_l"], params=vdn.Params(merge_mxfp8=1))
    b = vdn.attn_fwd(*args, gamma=t["gamma"], W_s=t["W_s"], W_l=t["W_l"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
