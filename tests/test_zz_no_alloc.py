"""The allocation-free Softmax entry point (vdn_window_softmax_fwd_noalloc)
against vdn_window_softmax_fwd, called through the C-ABI on the same inputs.

Both run the same kernels; only the scratch differs (the library's device
array instead of the caller's workspace), so outputs and lse must be equal
bit for bit.  Two calls in a row, the second on a smaller input, so the
second reads scratch the first one left behind; a size whose scratch exceeds
the array is rejected before any launch.
"""
import numpy as np
import pytest

from gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def _inputs(B, H, F, N, T, d, seed):
    import torch
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)
    L = F * N
    q, k, v = r(B, H, L, d), r(B, H, L, d), r(B, H, L, d)
    kt, vt = r(B, H, T, d), r(B, H, T, d)
    gs = torch.rand(B, H, L, generator=g).to(DEV)
    return q, k, v, kt, vt, gs


@pytest.mark.parametrize("text", [False, True])
def test_noalloc_matches_workspace_entry(text):
    import torch
    import softmax_attention_video_amd as vdn
    p = vdn.Params(text_softmax=int(text))
    # the small named shape, then a smaller ragged one (N % 64 != 0)
    for (B, H, F, N, T, d, seed) in ((1, 8, 60, 256, 64, 64, 1), (2, 2, 20, 80, 21, 128, 2)):
        log(f"[noalloc] text={text} B={B} H={H} F={F} N={N} T={T} d={d}")
        q, k, v, kt, vt, gs = _inputs(B, H, F, N, T, d, seed)
        L = F * N
        ref, ref_lse = vdn.window_softmax_fwd(q, k, v, F, g_s=gs, want_lse=True, params=p,
                                              k_text=kt, v_text=vt)
        out = torch.empty((B, L, H, d), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, H, L), dtype=torch.float32, device=DEV)
        vdn.window_softmax_fwd_noalloc(q, k, v, F, out, lse, g_s=gs, params=p, k_text=kt, v_text=vt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert torch.equal(lse, ref_lse)
        assert torch.isfinite(out.float()).all()


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import torch
    import softmax_attention_video_amd as vdn
    # V^T of 24 heads x 1536*120 tokens x 128 channels is 1.1 GB > 64 MiB:
    # the check runs on the host, nothing is launched (tiny tensors suffice
    # because shapes are only passed, never read)
    dims = vdn.Dims(1, 24, 120, 1536, 0, 128, 128, 24 * 128)
    pc = vdn.Params().c()
    x = torch.zeros(16, dtype=torch.bfloat16, device=DEV)
    import ctypes
    st = vdn.lib().vdn_window_softmax_fwd_noalloc(
        ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(x.data_ptr()),
        None, None, None, ctypes.c_void_p(x.data_ptr()), None, ctypes.byref(dims), ctypes.byref(pc),
        vdn.VDN_BF16, None)
    assert st == vdn.VDN_ERR_UNSUPPORTED
    assert b"64" in vdn.lib().vdn_last_error() or b"scratch" in vdn.lib().vdn_last_error()
    # fp32 storage runs the generic kernel, which needs no scratch at all
    need = vdn.lib().vdn_softmax_workspace_bytes(ctypes.byref(dims), ctypes.byref(pc), vdn.VDN_F32)
    assert need == 0
