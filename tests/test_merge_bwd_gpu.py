"""GPU parity of the merge backward (vdn_merge_bwd) against the fp64 oracle
(oracle/merge_bwd.py): d_ohat_s, d_ohat_l and dW_s, dW_l on seeded inputs of
several shapes (output columns not a multiple of the 256-wide tiles, two
batches), without weight gradients, identity projections, and the H3-scale
shape (B*L = 184320 tokens, H*d = D = 3072) on sampled rows and sampled
weight-gradient entries."""
import numpy as np
import pytest

from gpu_util import DEV, TOL, log, rel_l2, to_np
from oracle import merge_bwd as MB

pytestmark = pytest.mark.gpu


def _inputs(B, F, N, H, d, D, seed):
    import torch
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    L = F * N
    r = lambda *s, sc=1.0: (torch.randn(*s, generator=g, device=DEV) * sc).to(torch.bfloat16)
    return dict(os=r(B, L, H, d), ol=r(B, L, H, d), ws=r(H * d, D, sc=0.05), wl=r(H * d, D, sc=0.05),
                dout=r(B, L, D))


def _np(x):
    return to_np(x).astype(np.float64)


@pytest.mark.parametrize("B,F,N,H,d,D", [(1, 10, 128, 4, 64, 384), (2, 5, 64, 5, 32, 256), (1, 5, 256, 8, 64, 128)])
def test_merge_bwd_parity(B, F, N, H, d, D):
    import torch
    import softmax_attention_video_amd as vdn
    x = _inputs(B, F, N, H, d, D, seed=B * 100 + H)
    log(f"[merge-bwd] B={B} F={F} N={N} H={H} d={d} D={D}")
    dos, dol, dws, dwl = vdn.merge_bwd(x["dout"], x["os"], x["ol"], x["ws"], x["wl"], F)
    torch.cuda.synchronize()
    M, K = B * F * N, H * d
    ref = MB.merge_bwd(_np(x["os"]).reshape(M, K), _np(x["ol"]).reshape(M, K), _np(x["ws"]), _np(x["wl"]),
                       _np(x["dout"]).reshape(M, D))
    errs = [rel_l2(_np(g).reshape(r.shape), r) for g, r in zip((dos, dol, dws, dwl), ref)]
    log(f"[merge-bwd] rel-L2 dOs {errs[0]:.2e} dOl {errs[1]:.2e} dWs {errs[2]:.2e} dWl {errs[3]:.2e}")
    assert max(errs) <= TOL["bf16"], errs


def test_merge_bwd_without_weight_gradients_and_identity():
    import torch
    import softmax_attention_video_amd as vdn
    x = _inputs(1, 5, 64, 4, 32, 256, seed=7)          # B*L = 320: no weight gradients needed
    dos, dol, dws, dwl = vdn.merge_bwd(x["dout"], x["os"], x["ol"], x["ws"], x["wl"], 5, want_dw=False)
    torch.cuda.synchronize()
    assert dws is None and dwl is None
    ref = MB.merge_bwd(_np(x["os"]).reshape(320, 128), _np(x["ol"]).reshape(320, 128), _np(x["ws"]),
                       _np(x["wl"]), _np(x["dout"]).reshape(320, 256))
    assert rel_l2(_np(dos).reshape(320, 128), ref[0]) <= TOL["bf16"]
    assert rel_l2(_np(dol).reshape(320, 128), ref[1]) <= TOL["bf16"]
    # identity projections: D = H*d and the gradients are d_out itself
    dout = torch.randn((1, 320, 128), device=DEV).to(torch.bfloat16)
    dos, dol, dws, dwl = vdn.merge_bwd(dout, x["os"], x["ol"], None, None, 5)
    torch.cuda.synchronize()
    assert dws is None and torch.equal(dos.reshape(1, 320, 128), dout)
    assert torch.equal(dol.reshape(1, 320, 128), dout)


def test_merge_bwd_h3_sampled():
    """H3 shape in the configuration a training step would call: sampled rows
    of d_ohat_s / d_ohat_l and 64 sampled entries of dW_s / dW_l (each a sum
    over all 184320 tokens) against the oracle's definition."""
    import torch
    import softmax_attention_video_amd as vdn
    B, F, N, H, d, D = 1, 120, 1536, 24, 128, 3072
    x = _inputs(B, F, N, H, d, D, seed=11)
    log("[merge-bwd] h3: backward")
    dos, dol, dws, dwl = vdn.merge_bwd(x["dout"], x["os"], x["ol"], x["ws"], x["wl"], F)
    torch.cuda.synchronize()
    M, K = B * F * N, H * d
    rng = np.random.default_rng(5)
    rows = torch.from_numpy(np.sort(rng.choice(M, 24, replace=False))).to(DEV)
    dout_rows = _np(x["dout"].reshape(M, D).index_select(0, rows))
    for name, w, g in (("dOs", x["ws"], dos), ("dOl", x["wl"], dol)):
        ref = dout_rows @ _np(w).T
        e = rel_l2(_np(g.reshape(M, K).index_select(0, rows)), ref)
        log(f"[merge-bwd] h3 {name} sampled rows rel-L2 {e:.2e}")
        assert e <= TOL["bf16"]
    ii = rng.choice(K, 8, replace=False)
    jj = rng.choice(D, 8, replace=False)
    dcols = _np(x["dout"].reshape(M, D)[:, torch.from_numpy(jj).to(DEV)])          # [M, 8]
    for name, o, g in (("dWs", x["os"], dws), ("dWl", x["ol"], dwl)):
        ocols = _np(o.reshape(M, K)[:, torch.from_numpy(ii).to(DEV)])             # [M, 8]
        ref = ocols.T @ dcols                                                     # [8, 8]
        got = _np(g)[np.ix_(ii, jj)]
        e = rel_l2(got, ref)
        log(f"[merge-bwd] h3 {name} sampled entries rel-L2 {e:.2e}")
        assert e <= TOL["bf16"]
