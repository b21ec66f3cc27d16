"""C-ABI tests that need no GPU: exports, host-side argument checks, and the
frame-role tables of vdn_window_plan bit-exact against the oracle."""
import ctypes
import os
import re

import numpy as np
import pytest

import softmax_attention_video_amd as vdn
from oracle import vdn_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "vdn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b((?:vdn|vda)_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_header_symbol():
    L = vdn.lib()
    names = _header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(vdn.EXPORTS)


def test_default_params():
    p = vdn.default_params()
    assert (p.chunk_frames, p.window_chunks, p.anchors) == (5, 1, 1)
    assert p.text_init_scale == 0.5 and p.softmax_scale == 0.0 and p.text_softmax == 0
    assert abs(p.rms_eps - 1e-6) < 1e-12


def test_status_strings():
    L = vdn.lib()
    for code, name in [(0, b"VDN_OK"), (-1, b"VDN_ERR_INVALID_ARG"), (-2, b"VDN_ERR_UNSUPPORTED"),
                       (-3, b"VDN_ERR_WORKSPACE"), (-4, b"VDN_ERR_HIP")]:
        assert L.vdn_status_string(code) == name


PLAN_PARAMS = [O.Params(), O.Params(chunk_frames=3, window_chunks=2), O.Params(anchors=False),
               O.Params(chunk_frames=1, window_chunks=0), O.Params(chunk_frames=2, window_chunks=3),
               O.Params(chunk_frames=4, window_chunks=0, anchors=False),
               O.Params(chunk_frames=10, window_chunks=2)]


@pytest.mark.parametrize("F", list(range(2, 61)) + [100, 120, 240, 600])
@pytest.mark.parametrize("params", PLAN_PARAMS)
def test_window_plan_bit_exact(F, params):
    """vis comes from the Softmax kernels' work-item decoder run over their
    grid, the indices from the readout kernels' function: both bit-exact
    against the oracle's literal rule."""
    if F % params.chunk_frames:
        with pytest.raises(vdn.VdnError) as e:
            vdn.window_plan(F, vdn.Params(chunk_frames=params.chunk_frames))
        assert e.value.status == vdn.VDN_ERR_INVALID_ARG
        return
    vp = vdn.Params(chunk_frames=params.chunk_frames, window_chunks=params.window_chunks,
                    anchors=int(params.anchors))
    vis, i_f, ws, i_r, we = vdn.window_plan(F, vp)
    np.testing.assert_array_equal(vis, O.visibility(F, params))
    for got, exp in zip((i_f, ws, i_r, we), O.scan_indices(F, params)):
        np.testing.assert_array_equal(got, exp)


def _row_keys_expected(B, H, F, N, T, params: O.Params):
    vis = O.visibility(F, params).astype(np.int64)
    per_frame = vis.sum(axis=1) * N + (T if params.text_softmax else 0)
    return np.tile(np.repeat(per_frame, N), B * H)


@pytest.mark.parametrize("B,H,F,N,T,d,dt", [
    (1, 1, 20, 16, 8, 16, vdn.VDN_F32),          # tiny fp32 (generic kernel)
    (1, 8, 60, 256, 64, 64, vdn.VDN_BF16),       # small bf16 (MFMA kernel)
    (1, 16, 100, 384, 512, 128, vdn.VDN_BF16),   # medium
    (1, 24, 120, 1536, 512, 128, vdn.VDN_BF16),  # H3-scale layer
    (1, 16, 600, 768, 256, 128, vdn.VDN_BF16),   # long clip
    (2, 3, 20, 80, 5, 64, vdn.VDN_BF16),         # ragged tiles, two batches
    (1, 2, 10, 37, 3, 64, vdn.VDN_BF16),         # N % 16 != 0: generic kernel
    (1, 2, 35, 112, 21, 128, vdn.VDN_BF16),
    (3, 5, 15, 16, 0, 32, vdn.VDN_BF16),
])
@pytest.mark.parametrize("params", [O.Params(), O.Params(text_softmax=True), O.Params(anchors=False),
                                    O.Params(chunk_frames=3, window_chunks=2, text_softmax=True),
                                    O.Params(chunk_frames=1, window_chunks=0, anchors=False)])
def test_window_row_keys_bit_exact(B, H, F, N, T, d, dt, params):
    """Every query row of every head is covered by exactly one work item of
    the forward Softmax launch, and that item walks exactly N*|Vis(t)| video
    keys (+ T text keys with text_softmax): the launch's own decoder, run over
    its whole grid, against the oracle's visibility rule."""
    if F % params.chunk_frames:
        pytest.skip("F not a multiple of chunk_frames")
    dims = vdn.Dims(B, H, F, N, T, d, d, H * d)
    vp = vdn.Params(chunk_frames=params.chunk_frames, window_chunks=params.window_chunks,
                    anchors=int(params.anchors), text_softmax=int(params.text_softmax))
    got = vdn.window_row_keys(dims, vp, dt)
    np.testing.assert_array_equal(got, _row_keys_expected(B, H, F, N, T, params))


def test_window_row_keys_rejects_bad_args():
    L = vdn.lib()
    p = vdn.Params().c()
    keys = np.zeros(20 * 16, np.int64)
    assert L.vdn_window_row_keys(ctypes.byref(_dims(F=22)), ctypes.byref(p), vdn.VDN_BF16,
                                 keys.ctypes.data) == vdn.VDN_ERR_INVALID_ARG
    assert L.vdn_window_row_keys(ctypes.byref(_dims()), ctypes.byref(p), vdn.VDN_BF16,
                                 None) == vdn.VDN_ERR_INVALID_ARG


def test_window_plan_rejects_bad_args():
    with pytest.raises(vdn.VdnError):
        vdn.window_plan(1)
    with pytest.raises(vdn.VdnError):
        vdn.window_plan(20, vdn.Params(anchors=2))


# ---- argument validation: every failing check returns before any HIP call ----
def _call_attn(dims, params=None, dt=vdn.VDN_BF16, ws_bytes=1 << 40, null=(), W=True):
    L = vdn.lib()
    p = (params or vdn.Params()).c()
    fake = ctypes.c_void_p(0x100000)
    ptrs = [fake] * 16
    names = ["q", "k", "v", "beta", "alpha", "k_text", "v_text", "beta_text", "g_s", "g_l",
             "gamma", "W_s", "W_l", "out", "ohat_s", "ohat_l"]
    for n in null:
        ptrs[names.index(n)] = None
    if not W:
        ptrs[names.index("W_s")] = ptrs[names.index("W_l")] = None
    return L.vdn_attn_fwd(*ptrs, fake, ctypes.c_size_t(ws_bytes),
                          ctypes.byref(dims) if dims is not None else None,
                          ctypes.byref(p), dt, None)


def _dims(**kw):
    d = dict(B=1, H=2, F=20, N=16, T=4, d_k=64, d_v=64, D=128)
    d.update(kw)
    return vdn.Dims(*[d[k] for k in ("B", "H", "F", "N", "T", "d_k", "d_v", "D")])


@pytest.mark.parametrize("kw,code", [
    (dict(F=1), vdn.VDN_ERR_INVALID_ARG),
    (dict(F=22), vdn.VDN_ERR_INVALID_ARG),          # not a multiple of 5
    (dict(N=0), vdn.VDN_ERR_INVALID_ARG),
    (dict(B=0), vdn.VDN_ERR_INVALID_ARG),
    (dict(H=0), vdn.VDN_ERR_INVALID_ARG),
    (dict(T=-1), vdn.VDN_ERR_INVALID_ARG),
    (dict(D=0), vdn.VDN_ERR_INVALID_ARG),
    (dict(d_k=48, d_v=48), vdn.VDN_ERR_UNSUPPORTED),
    (dict(d_k=64, d_v=32), vdn.VDN_ERR_UNSUPPORTED),
    (dict(d_k=256, d_v=256), vdn.VDN_ERR_UNSUPPORTED),
])
def test_attn_invalid_dims(kw, code):
    assert _call_attn(_dims(**kw)) == code
    assert vdn.lib().vdn_last_error() != b""


def test_attn_null_pointers_and_pairs():
    assert _call_attn(None) == vdn.VDN_ERR_INVALID_ARG
    for n in ("q", "k", "v", "beta", "alpha", "g_s", "g_l", "out", "k_text", "v_text",
              "beta_text"):
        assert _call_attn(_dims(), null=(n,)) == vdn.VDN_ERR_INVALID_ARG, n
    # only one projection
    assert _call_attn(_dims(), null=("W_l",)) == vdn.VDN_ERR_INVALID_ARG
    # identity merge needs D == H * d_v
    assert _call_attn(_dims(D=100), W=False) == vdn.VDN_ERR_INVALID_ARG


def test_attn_unknown_dtype_and_params():
    assert _call_attn(_dims(), dt=7) == vdn.VDN_ERR_UNSUPPORTED
    assert _call_attn(_dims(), params=vdn.Params(chunk_frames=0)) == vdn.VDN_ERR_INVALID_ARG
    assert _call_attn(_dims(), params=vdn.Params(window_chunks=-1)) == vdn.VDN_ERR_INVALID_ARG
    assert _call_attn(_dims(), params=vdn.Params(rms_eps=-1.0)) == vdn.VDN_ERR_INVALID_ARG


def test_attn_workspace_too_small():
    d = _dims()
    need = vdn.workspace_bytes(d)
    assert need > 0
    # without caller buffers for the branch outputs the whole layout is needed
    assert _call_attn(d, ws_bytes=need - 1, null=("ohat_s", "ohat_l")) == vdn.VDN_ERR_WORKSPACE
    assert _call_attn(d, ws_bytes=need - 1, null=("ohat_s",)) == vdn.VDN_ERR_WORKSPACE
    # with both given, their two regions (last in the layout) are not needed
    oh = 2 * ((d.B * d.H * d.F * d.N * d.d_v * 2 + 255) // 256 * 256)
    assert _call_attn(d, ws_bytes=need - oh - 1) == vdn.VDN_ERR_WORKSPACE


def test_per_entry_workspace_queries():
    """Each entry point needs only its own regions: the scan its frame maps
    (and chunk maps for d = 16, 32), the Softmax the transposed values (bf16
    MFMA path), the merge the transposed projections."""
    L = vdn.lib()
    p = vdn.Params()
    pc = p.c()
    for d_ in (32, 64):
        d = _dims(d_k=d_, d_v=d_, D=2 * d_)
        BH, F, C, DD = d.B * d.H, d.F, d.F // 5, d_ * d_
        a256 = lambda x: (x + 255) // 256 * 256
        scan = L.vdn_scan_workspace_bytes(ctypes.byref(d), ctypes.byref(pc), vdn.VDN_BF16)
        maps = 2 * a256(BH * F * DD * 4) + a256(BH * DD * 4)
        chunks = 2 * a256(BH * 2 * C * DD * 4) if d_ == 32 else 0
        assert scan == maps + chunks
        sm = L.vdn_softmax_workspace_bytes(ctypes.byref(d), ctypes.byref(pc), vdn.VDN_BF16)
        assert sm == (a256(BH * d.F * d.N * d_ * 2) if d_ == 64 else 0)   # MFMA path: d = 64, 128
        assert L.vdn_softmax_workspace_bytes(ctypes.byref(d), ctypes.byref(pc), vdn.VDN_F32) == 0
        mg = L.vdn_merge_workspace_bytes(ctypes.byref(d), ctypes.byref(pc), vdn.VDN_BF16)
        assert mg == 2 * a256(d.H * d_ * d.D * 2)
        assert max(scan, sm, mg) < vdn.workspace_bytes(d, p)
        fake = ctypes.c_void_p(0x100000)
        for fn in (L.vda_scan_fwd, L.vda_scan_rev):
            assert fn(*[fake] * 9, fake, ctypes.c_size_t(scan - 1), ctypes.byref(d), ctypes.byref(pc),
                      vdn.VDN_BF16, None) == vdn.VDN_ERR_WORKSPACE
        if sm > 0:    # (a call that passes the check would launch kernels on fake pointers)
            assert L.vdn_window_softmax_fwd(fake, fake, fake, None, None, None, fake, None, fake,
                                            ctypes.c_size_t(sm - 1), ctypes.byref(d), ctypes.byref(pc),
                                            vdn.VDN_BF16, None) == vdn.VDN_ERR_WORKSPACE
        assert L.vdn_merge_fwd(fake, fake, fake, fake, fake, fake, ctypes.c_size_t(mg - 1),
                               ctypes.byref(d), ctypes.byref(pc), vdn.VDN_BF16, None) == vdn.VDN_ERR_WORKSPACE
    bad = _dims(F=21)
    for fn in (L.vdn_scan_workspace_bytes, L.vdn_softmax_workspace_bytes, L.vdn_merge_workspace_bytes):
        assert fn(ctypes.byref(bad), ctypes.byref(pc), vdn.VDN_BF16) == 0


def test_workspace_bytes_zero_for_invalid():
    assert vdn.workspace_bytes(_dims(F=21)) == 0
    assert vdn.workspace_bytes(_dims(d_k=48, d_v=48)) == 0


def test_scan_and_softmax_validation():
    L = vdn.lib()
    p = vdn.Params().c()
    fake = ctypes.c_void_p(0x100000)
    d = _dims()
    for fn in (L.vda_scan_fwd, L.vda_scan_rev):
        # no output state
        assert fn(*[fake] * 7, None, None, fake, ctypes.c_size_t(1 << 40), ctypes.byref(d),
                  ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG
        # workspace too small
        assert fn(*[fake] * 9, fake, ctypes.c_size_t(16), ctypes.byref(d), ctypes.byref(p),
                  vdn.VDN_BF16, None) == vdn.VDN_ERR_WORKSPACE
    sm = L.vdn_window_softmax_fwd
    assert sm(None, fake, fake, None, None, None, fake, None, fake, ctypes.c_size_t(1 << 40),
              ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG
    assert sm(fake, fake, fake, None, None, None, fake, None, fake, ctypes.c_size_t(16),
              ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_WORKSPACE
    # text keys inside the Softmax: both text pointers are required when T > 0
    pt = vdn.Params(text_softmax=1).c()
    for kt, vt in ((None, fake), (fake, None)):
        assert sm(fake, fake, fake, kt, vt, None, fake, None, fake, ctypes.c_size_t(1 << 40),
                  ctypes.byref(d), ctypes.byref(pt), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG
    # ... and not read without the option (T > 0, NULL text, workspace check reached)
    assert sm(fake, fake, fake, None, None, None, fake, None, fake, ctypes.c_size_t(16),
              ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_WORKSPACE
    assert d.T > 0
    # text_softmax must be 0 or 1
    assert _call_attn(_dims(), params=vdn.Params(text_softmax=2)) == vdn.VDN_ERR_INVALID_ARG


def test_text_softmax_workspace_holds_padded_text_columns():
    # bf16 MFMA path: V^T of a head spans L video + T text columns rounded up to 16
    d = _dims(B=1, H=2, F=20, N=16, T=5, d_k=64, d_v=64, D=128)
    base = vdn.workspace_bytes(d, vdn.Params())
    text = vdn.workspace_bytes(d, vdn.Params(text_softmax=1))
    assert text >= base + 2 * 64 * 16 * 2 - 256
    assert text <= base + 2 * 64 * 16 * 2 + 256
    d0 = _dims(B=1, H=2, F=20, N=16, T=0, d_k=64, d_v=64, D=128)
    assert vdn.workspace_bytes(d0, vdn.Params(text_softmax=1)) == vdn.workspace_bytes(d0)


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 20, 16)
    with pytest.raises(ValueError):
        vdn.window_softmax_fwd(q, q, q, F=20)


def _call_prep(dims, params, null=(), dt=vdn.VDN_BF16):
    L = vdn.lib()
    fake = ctypes.c_void_p(0x100000)
    names = ("q", "k", "v", "w_spatial", "w_temporal", "q_out", "k_out", "v_out")
    args = [None if n in null else fake for n in names]
    return L.vda_prep_fwd(*args, ctypes.byref(dims) if dims is not None else None,
                          ctypes.byref(params) if params is not None else None, dt, None)


def test_prep_default_params():
    p = vdn.CPrepParams()
    vdn.lib().vda_prep_default_params(ctypes.byref(p), 48, 32)
    assert (p.grid_h, p.grid_w, p.kernel_h, p.kernel_w, p.taps, p.causal) == (48, 32, 3, 3, 5, 0)
    assert abs(p.l2_eps - 1e-6) < 1e-12
    c = vdn.PrepParams(48, 32).c()
    assert (c.kernel_h, c.kernel_w, c.taps, c.causal) == (3, 3, 5, 0)


@pytest.mark.parametrize("dkw,pkw,code", [
    (dict(), dict(grid_h=4, grid_w=5), vdn.VDN_ERR_INVALID_ARG),             # N != grid_h * grid_w
    (dict(d_k=48, d_v=48), dict(), vdn.VDN_ERR_UNSUPPORTED),
    (dict(d_k=64, d_v=32), dict(), vdn.VDN_ERR_UNSUPPORTED),
    (dict(F=0), dict(), vdn.VDN_ERR_INVALID_ARG),
    (dict(B=0), dict(), vdn.VDN_ERR_INVALID_ARG),
    (dict(), dict(kernel_h=2), vdn.VDN_ERR_UNSUPPORTED),
    (dict(), dict(kernel_w=9), vdn.VDN_ERR_UNSUPPORTED),
    (dict(), dict(taps=6), vdn.VDN_ERR_UNSUPPORTED),
    (dict(), dict(taps=0), vdn.VDN_ERR_UNSUPPORTED),
    (dict(), dict(causal=2), vdn.VDN_ERR_INVALID_ARG),
    (dict(), dict(l2_eps=-1.0), vdn.VDN_ERR_INVALID_ARG),
])
def test_prep_invalid_args(dkw, pkw, code):
    base = dict(B=1, H=2, F=4, N=16, T=0, d_k=64, d_v=64, D=128)
    base.update(dkw)
    d = vdn.Dims(*(base[k] for k in ("B", "H", "F", "N", "T", "d_k", "d_v", "D")))
    pp = dict(grid_h=4, grid_w=4)
    pp.update(pkw)
    assert _call_prep(d, vdn.PrepParams(**pp).c()) == code
    assert vdn.lib().vdn_last_error() != b""


def test_prep_null_pointers_and_dtype():
    d = vdn.Dims(1, 2, 4, 16, 0, 64, 64, 128)
    p = vdn.PrepParams(4, 4).c()
    assert _call_prep(None, p) == vdn.VDN_ERR_INVALID_ARG
    assert _call_prep(d, None) == vdn.VDN_ERR_INVALID_ARG
    for n in ("q", "k", "v", "w_spatial", "w_temporal", "q_out", "k_out", "v_out"):
        assert _call_prep(d, p, null=(n,)) == vdn.VDN_ERR_INVALID_ARG, n
    assert _call_prep(d, p, dt=7) == vdn.VDN_ERR_UNSUPPORTED


def test_mx_merge_validation():
    d = _dims()
    assert _call_attn(d, params=vdn.Params(merge_mxfp8=2)) == vdn.VDN_ERR_INVALID_ARG
    assert _call_attn(d, params=vdn.Params(merge_mxfp8=1), dt=vdn.VDN_F32) == vdn.VDN_ERR_UNSUPPORTED
    assert _call_attn(d, params=vdn.Params(merge_mxfp8=1), W=False) == vdn.VDN_ERR_INVALID_ARG
    # H * d_v must be a multiple of 64 (128-deep K steps over the concatenated K)
    assert _call_attn(_dims(H=1, d_k=32, d_v=32, D=32),
                      params=vdn.Params(merge_mxfp8=1)) == vdn.VDN_ERR_UNSUPPORTED
    assert _call_attn(_dims(D=130), params=vdn.Params(merge_mxfp8=1)) == vdn.VDN_ERR_UNSUPPORTED


def test_mx_workspace_holds_codes_and_scales():
    d = _dims(B=1, H=2, F=20, N=16, T=4, d_k=64, d_v=64, D=96)
    base = vdn.workspace_bytes(d, vdn.Params())
    mx = vdn.workspace_bytes(d, vdn.Params(merge_mxfp8=1))
    M, K2, Dm = 20 * 16, 2 * 128, 96
    extra = M * K2 + M * K2 // 32 + Dm * K2 + Dm * K2 // 32
    assert extra <= mx - base <= extra + 4 * 256
    # fp32 storage never uses the MX operands
    assert vdn.workspace_bytes(d, vdn.Params(merge_mxfp8=1), vdn.VDN_F32) == \
        vdn.workspace_bytes(d, vdn.Params(), vdn.VDN_F32)


def test_merge_fwd_and_quantize_validation():
    L = vdn.lib()
    fake = ctypes.c_void_p(0x100000)
    d = _dims()
    p = vdn.Params().c()
    pm = vdn.Params(merge_mxfp8=1).c()
    big = ctypes.c_size_t(1 << 40)
    assert L.vdn_merge_fwd(None, fake, fake, fake, fake, fake, big, ctypes.byref(d), ctypes.byref(p),
                           vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG
    assert L.vdn_merge_fwd(fake, fake, fake, None, fake, fake, big, ctypes.byref(d), ctypes.byref(p),
                           vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG
    assert L.vdn_merge_fwd(fake, fake, fake, fake, fake, fake, ctypes.c_size_t(16), ctypes.byref(d),
                           ctypes.byref(pm), vdn.VDN_BF16, None) == vdn.VDN_ERR_WORKSPACE
    assert L.vdn_merge_fwd(fake, fake, None, None, fake, fake, big, ctypes.byref(d), ctypes.byref(pm),
                           vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG
    q = L.vdn_mx_quantize
    assert q(None, fake, fake, 4, 64, None) == vdn.VDN_ERR_INVALID_ARG
    assert q(fake, fake, None, 4, 64, None) == vdn.VDN_ERR_INVALID_ARG
    assert q(fake, fake, fake, 4, 48, None) == vdn.VDN_ERR_INVALID_ARG
    assert b"multiple of 32" in L.vdn_last_error()
    assert q(fake, fake, fake, -1, 64, None) == vdn.VDN_ERR_INVALID_ARG


def test_softmax_bwd_validation():
    """Host-side checks of vdn_window_softmax_bwd: required pointers (the
    text ones only with text keys), workspace size and the workspace query."""
    L = vdn.lib()
    fake = ctypes.c_void_p(0x100000)
    d = _dims()                       # T = 4
    p = vdn.Params().c()
    big = ctypes.c_size_t(1 << 40)
    # q k v k_text v_text o lse g_s d_out dq dk dv dk_text dv_text dg_s
    args = [fake] * 15
    fn = L.vdn_window_softmax_bwd
    for i in (0, 1, 2, 5, 6, 8, 9, 10, 11):
        a = list(args)
        a[i] = None
        assert fn(*a, fake, big, ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG, i
    # without text keys the text pointers, g_s and dg_s may be NULL
    a = list(args)
    for i in (3, 4, 7, 12, 13, 14):
        a[i] = None
    assert fn(*a, fake, ctypes.c_size_t(16), ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16,
              None) == vdn.VDN_ERR_WORKSPACE
    # with text keys they are required
    pt = vdn.Params(text_softmax=1).c()
    for i in (3, 4, 12, 13):
        a = list(args)
        a[i] = None
        assert fn(*a, fake, big, ctypes.byref(d), ctypes.byref(pt), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG, i
    assert fn(*args, fake, ctypes.c_size_t(16), ctypes.byref(d), ctypes.byref(pt), vdn.VDN_BF16,
              None) == vdn.VDN_ERR_WORKSPACE
    need = L.vdn_softmax_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16)
    assert need >= 2 * 20 * 16 * 64 * 2 + 2 * 20 * 16 * 4
    need_t = L.vdn_softmax_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(pt), vdn.VDN_BF16)
    assert need_t >= need


def test_vda_bwd_validation():
    """Host-side checks of vda_bwd: required pointers, text pointers when
    T > 0, workspace size, the frame limit, and the workspace query."""
    L = vdn.lib()
    fake = ctypes.c_void_p(0x100000)
    d = _dims()                       # T = 4
    p = vdn.Params().c()
    big = ctypes.c_size_t(1 << 40)
    args = [fake] * 21                # q k v beta alpha k_text v_text beta_text g_l gamma d_out dq dk dv
    fn = L.vda_bwd                    # dbeta dalpha dk_text dv_text dbeta_text dg_l dgamma
    for i in (0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 12, 13, 14, 15, 16, 17, 18):
        a = list(args)
        a[i] = None
        assert fn(*a, fake, big, ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG, i
    for i in (9, 19, 20):             # gamma, dg_l, dgamma are optional: the call gets past the checks
        a = list(args)
        a[i] = None
        assert fn(*a, fake, ctypes.c_size_t(16), ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16,
                  None) == vdn.VDN_ERR_WORKSPACE, i
    d0 = _dims()
    d0.T = 0                          # no text: its pointers may be NULL
    a = list(args)
    for i in (5, 6, 7, 16, 17, 18):
        a[i] = None
    assert fn(*a, fake, ctypes.c_size_t(16), ctypes.byref(d0), ctypes.byref(p), vdn.VDN_BF16,
              None) == vdn.VDN_ERR_WORKSPACE
    dbig = _dims()
    dbig.F, dbig.N = 1030, 1          # 206 chunks of 5: beyond the frame limit
    assert fn(*args, fake, big, ctypes.byref(dbig), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_UNSUPPORTED
    need = L.vda_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16)
    BH, F, D, C = d.B * d.H, d.F, d.d_k, d.F // 5
    assert need >= 4 * BH * D * D * (3 * F + 1 + 4 * C + 2 * (C + 1) + F + 4 * (C + 1) + 2 * (F + 1) + 2 * F)
    bad = _dims()
    bad.d_k = bad.d_v = 48
    assert L.vda_bwd_workspace_bytes(ctypes.byref(bad), ctypes.byref(p), vdn.VDN_BF16) == 0


def test_merge_bwd_validation():
    """Host-side checks of vdn_merge_bwd: required pointers, paired W and dW,
    the supported storage and shapes, the workspace, and its query."""
    L = vdn.lib()
    fake = ctypes.c_void_p(0x100000)
    d = _dims(N=32, D=256)           # B*L = 640, a multiple of 128
    p = vdn.Params().c()
    big = ctypes.c_size_t(1 << 40)
    args = [fake] * 9                 # ohat_s ohat_l W_s W_l d_out d_ohat_s d_ohat_l dW_s dW_l
    fn = L.vdn_merge_bwd
    for i in (4, 5, 6):
        a = list(args)
        a[i] = None
        assert fn(*a, fake, big, ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG, i
    for i in (2, 7):                  # unpaired W or dW
        a = list(args)
        a[i] = None
        assert fn(*a, fake, big, ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG, i
    assert fn(*args, fake, big, ctypes.byref(d), ctypes.byref(p), vdn.VDN_F32, None) == vdn.VDN_ERR_UNSUPPORTED
    d_odd = _dims(D=200)
    assert fn(*args, fake, big, ctypes.byref(d_odd), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_UNSUPPORTED
    assert fn(*args, fake, ctypes.c_size_t(16), ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16,
              None) == vdn.VDN_ERR_WORKSPACE
    need = L.vdn_merge_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16)
    assert need >= (20 * 32) * (256 + 128) * 2
    d_rag = _dims(D=256)              # B*L = 320: no weight gradients for it
    assert fn(*args, fake, big, ctypes.byref(d_rag), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_UNSUPPORTED


def test_noalloc_softmax_validation():
    """Host-side checks of vdn_window_softmax_fwd_noalloc: required pointers,
    text pointers with text keys, and sizes beyond its scratch array, all
    rejected before any HIP call."""
    L = vdn.lib()
    fake = ctypes.c_void_p(0x100000)
    d = _dims()
    p = vdn.Params().c()
    fn = L.vdn_window_softmax_fwd_noalloc
    # q k v k_text v_text g_s out lse
    for i in (0, 1, 2, 6):
        a = [fake] * 8
        a[i] = None
        assert fn(*a, ctypes.byref(d), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG, i
    pt = vdn.Params(text_softmax=1).c()
    for i in (3, 4):
        a = [fake] * 8
        a[i] = None
        assert fn(*a, ctypes.byref(d), ctypes.byref(pt), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG, i
    assert fn(*[fake] * 8, None, ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_INVALID_ARG
    assert fn(*[fake] * 8, ctypes.byref(d), ctypes.byref(p), 7, None) == vdn.VDN_ERR_UNSUPPORTED
    big = vdn.Dims(1, 24, 120, 1536, 0, 128, 128, 24 * 128)     # V^T of 1.1 GB
    assert fn(*[fake] * 8, ctypes.byref(big), ctypes.byref(p), vdn.VDN_BF16, None) == vdn.VDN_ERR_UNSUPPORTED
    assert b"scratch" in L.vdn_last_error()
