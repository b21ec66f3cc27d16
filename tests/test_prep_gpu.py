"""GPU parity of vda_prep_fwd (the linear branch's feature map, VDA-Prep)
against the fp64 oracle: whole tensors at the tiny and small sizes, filter
variants and a ragged grid, and sampled token rows of every output at the
medium, H3-scale and long-clip sizes (plus the unit norm of every k' row)."""
import numpy as np
import pytest

from gpu_util import DEV, log, rel_l2, to_np
from oracle import vda_prep as OP
from vdn_inputs import CONFIGS, GRIDS, prep_filters, prep_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}

VARIANTS = {
    "default": dict(),
    "causal": dict(causal=1),
    "k1x1": dict(kernel_h=1, kernel_w=1),
    "k5x3_t3": dict(kernel_h=5, kernel_w=3, taps=3),
    "k3x5_t1": dict(kernel_h=3, kernel_w=5, taps=1),
    "k7x7": dict(kernel_h=7, kernel_w=7),
}


def _device_inputs(cfg, inp, ws, wt):
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    # the feature map reads token-major [B, L, H, d]; the generator is [B, H, L, d]
    tm = [torch.from_numpy(inp[x]).to(DEV).permute(0, 2, 1, 3).contiguous().to(dt) for x in ("q", "k", "v")]
    return tm, torch.from_numpy(ws).to(DEV), torch.from_numpy(wt).to(DEV)


def _run(cfg, params, inp, ws, wt):
    import torch
    import softmax_attention_video_amd as vdn
    (q, k, v), wsd, wtd = _device_inputs(cfg, inp, ws, wt)
    out = vdn.prep_fwd(q, k, v, wsd, wtd, cfg.F, params)
    torch.cuda.synchronize()
    return out


def _oracle_params(p):
    return OP.PrepParams(p.grid_h, p.grid_w, p.kernel_h, p.kernel_w, p.taps, bool(p.causal), p.l2_eps)


def _check_full(cfg, params, tag):
    import softmax_attention_video_amd as vdn   # noqa: F401  (library must load)
    ws, wt = prep_filters(cfg, params.kernel_h, params.kernel_w, params.taps)
    inp = prep_inputs(cfg)
    log(f"[prep] {tag}: B={cfg.B} H={cfg.H} d={cfg.d} F={cfg.F} grid={params.grid_h}x{params.grid_w}")
    got = [to_np(x) for x in _run(cfg, params, inp, ws, wt)]
    op = _oracle_params(params)
    for b in range(cfg.B):
        for h in range(cfg.H):
            exp = OP.prep_head(inp["q"][b, h].astype(np.float64), inp["k"][b, h].astype(np.float64),
                               inp["v"][b, h].astype(np.float64), ws[h].astype(np.float64),
                               wt[h].astype(np.float64), op)
            for name, g, e in zip(("q'", "k'", "v'"), got, exp):
                err = rel_l2(g[b, h], e)
                assert err <= TOL[cfg.dtype], f"{tag} {name} b={b} h={h}: rel-L2 {err:.3e}"
    log(f"[prep] {tag}: ok")


@pytest.mark.parametrize("name", ["tiny", "small"])
@pytest.mark.parametrize("variant", list(VARIANTS))
def test_prep_parity_full(name, variant):
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS[name]
    gh, gw = GRIDS[name]
    _check_full(cfg, vdn.PrepParams(gh, gw, **VARIANTS[variant]), f"{name}/{variant}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prep_ragged_grid(dtype):
    """A grid wider than one column tile with a partial last tile, a short
    clip (F smaller than the temporal filter) and a non-square filter."""
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS["tiny"].replace(name="ragged", dtype=dtype, B=2, H=3, d=32, F=3, N=5 * 37)
    _check_full(cfg, vdn.PrepParams(5, 37, kernel_h=3, kernel_w=5), f"ragged/{dtype}")


def _sample_rows(cfg, gh, gw, n_random=96, seed=0):
    N, F = cfg.N, cfg.F
    rows = set()
    for f in (0, 1, 2, F // 2, F - 3, F - 2, F - 1):
        for n in (0, gw - 1, N - gw, N - 1, (gh // 2) * gw + gw // 2, gw, 2 * gw - 1):
            rows.add(f * N + n)
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.choice(cfg.L, size=n_random, replace=False))
    return np.array(sorted(rows), np.int64)


@pytest.mark.parametrize("name", ["medium", "h3", "long"])
def test_prep_full_size_sampled(name):
    import torch
    import softmax_attention_video_amd as vdn
    cfg = CONFIGS[name]
    gh, gw = GRIDS[name]
    params = vdn.PrepParams(gh, gw)
    ws, wt = prep_filters(cfg)
    log(f"[prep-large] {name}: generating inputs")
    inp = prep_inputs(cfg)
    log(f"[prep-large] {name}: running vda_prep_fwd")
    qo, ko, vo = _run(cfg, params, inp, ws, wt)
    # every k' row has unit norm up to bf16 rounding (a property at any size)
    nk = torch.linalg.vector_norm(ko.float(), dim=-1)
    assert float((nk - 1.0).abs().max()) < 1e-2, f"{name}: k' row norms off by {float((nk - 1).abs().max()):.3e}"
    op = _oracle_params(params)
    rows = _sample_rows(cfg, gh, gw)
    rt = torch.from_numpy(rows).to(DEV)
    for h in (0, cfg.H - 1):
        b = 0
        k64 = inp["k"][b, h].astype(np.float64)
        v64 = inp["v"][b, h].astype(np.float64)
        ek, ev = OP.prep_rows(k64, v64, ws[h].astype(np.float64), wt[h].astype(np.float64), rows, op)
        eq = OP.l2_normalize(inp["q"][b, h][rows].astype(np.float64), op.l2_eps)
        for tag, g, e in (("q'", qo, eq), ("k'", ko, ek), ("v'", vo, ev)):
            err = rel_l2(to_np(g[b, h].index_select(0, rt)), e)
            log(f"[prep-large] {name} h={h} {tag}: rel-L2 {err:.3e}")
            assert err <= TOL[cfg.dtype], f"{name} h={h} {tag}: rel-L2 {err:.3e}"
