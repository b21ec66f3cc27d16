"""Exact visible-key count of every query row, read from the GPU kernels.

With q = 0 every logit is 0, so each row's softmax is uniform over the keys
its work item walks and lse = ln(#keys).  round(exp(lse)) must equal
N * |Vis(t)| (+ T with text keys in the Softmax) for every row of every head:
the oracle's visibility rule (method, local Softmax window and boundary
anchors), checked bit-exactly on the masks and spans the kernels actually
use -- including the masked tails of partial key blocks.
"""
import numpy as np
import pytest

from oracle import vdn_oracle as O
from gpu_util import DEV, log

pytestmark = pytest.mark.gpu


def _expected(F, N, T, p: O.Params):
    vis = O.visibility(F, p).astype(np.int64)
    per_frame = vis.sum(axis=1) * N + (T if p.text_softmax else 0)
    return np.repeat(per_frame, N)


@pytest.mark.parametrize("F", [20, 60, 120, 600])
@pytest.mark.parametrize("text", [False, True])
@pytest.mark.parametrize("anchors", [True, False])
@pytest.mark.parametrize("path", ["bf16_mfma", "f32"])
def test_lse_counts_visible_keys(F, text, anchors, path):
    import torch
    import softmax_attention_video_amd as vdn
    B, H, N, T = 1, 2, 16, 21
    d = 64 if path == "bf16_mfma" else 16
    dt = torch.bfloat16 if path == "bf16_mfma" else torch.float32
    p = O.Params(anchors=anchors, text_softmax=text)
    vp = vdn.Params(anchors=int(anchors), text_softmax=int(text))
    log(f"[count] F={F} text={text} anchors={anchors} path={path}")
    g = torch.Generator().manual_seed(F)
    L = F * N
    q = torch.zeros(B, H, L, d, dtype=dt, device=DEV)
    k = torch.randn(B, H, L, d, generator=g).to(dt).to(DEV)
    v = torch.randn(B, H, L, d, generator=g).to(dt).to(DEV)
    kt = torch.randn(B, H, T, d, generator=g).to(dt).to(DEV)
    vt = torch.randn(B, H, T, d, generator=g).to(dt).to(DEV)
    _, lse = vdn.window_softmax_fwd(q, k, v, F, want_lse=True, params=vp, k_text=kt, v_text=vt)
    torch.cuda.synchronize()
    cnt = torch.exp(lse.double()).cpu().numpy()
    exp = _expected(F, N, T, p)
    for b in range(B):
        for h in range(H):
            got = np.rint(cnt[b, h]).astype(np.int64)
            bad = np.nonzero(got != exp)[0]
            assert bad.size == 0, (b, h, bad[:8], got[bad[:8]], exp[bad[:8]])
            # the count is an exact integer in fp32 (well below 2^24)
            assert np.abs(cnt[b, h] - exp).max() <= 1e-4 * exp.max()
