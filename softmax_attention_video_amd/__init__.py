"""MI355X-native Video DeltaNet (VDN) attention forward.

A thin ctypes binding over the HIP library libvdn.so (C-ABI in include/vdn.h).
Every step of the operator runs in the library's gfx950 kernels; this module
only checks tensor shapes/dtypes, allocates the workspace through torch and
passes raw device pointers and the current stream.  There is no fallback: if
the library is missing, every call raises.

Entry points (same names as the C-ABI):
  attn_fwd(...)               -> out            (vdn_attn_fwd)
  scan_fwd(...), scan_rev(...) -> P, S_text     (vda_scan_fwd / vda_scan_rev)
  window_softmax_fwd(...)     -> out, lse       (vdn_window_softmax_fwd)
  window_softmax_bwd(...)     -> dq, dk, dv, dg (vdn_window_softmax_bwd)
  merge_fwd(...)              -> out            (vdn_merge_fwd)
  mx_quantize(x)              -> codes, scales  (vdn_mx_quantize)
  prep_fwd(...)               -> q', k', v'     (vda_prep_fwd)
  window_plan(F, params)      -> host tables    (vdn_window_plan)
  window_row_keys(dims, ...)  -> keys per row   (vdn_window_row_keys)
  workspace_bytes(...)
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# VDN_LIB overrides the library path (the host-sanitizer test loads its
# instrumented build this way); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("VDN_LIB") or os.path.join(_HERE, "libvdn.so")

VDN_OK, VDN_ERR_INVALID_ARG, VDN_ERR_UNSUPPORTED, VDN_ERR_WORKSPACE, VDN_ERR_HIP = 0, -1, -2, -3, -4
VDN_F32, VDN_BF16 = 0, 1

EXPORTS = ("vdn_default_params", "vdn_attn_fwd", "vda_scan_fwd", "vda_scan_rev",
           "vdn_window_softmax_fwd", "vdn_workspace_bytes", "vdn_window_plan",
           "vdn_status_string", "vdn_last_error", "vdn_timer_enable", "vdn_timer_read",
           "vdn_timer_disable", "vda_prep_default_params", "vda_prep_fwd", "vdn_merge_fwd",
           "vdn_mx_quantize", "vdn_window_softmax_bwd", "vdn_softmax_bwd_workspace_bytes",
           "vda_bwd", "vda_bwd_workspace_bytes", "vdn_merge_bwd", "vdn_merge_bwd_workspace_bytes",
           "vdn_window_row_keys", "vdn_scan_workspace_bytes", "vdn_softmax_workspace_bytes",
           "vdn_merge_workspace_bytes", "vdn_window_softmax_fwd_noalloc")


class VdnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("B", "H", "F", "N", "T", "d_k", "d_v", "D")]


class CParams(ctypes.Structure):
    _fields_ = [("softmax_scale", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("text_init_scale", ctypes.c_float), ("chunk_frames", ctypes.c_int),
                ("window_chunks", ctypes.c_int), ("anchors", ctypes.c_int),
                ("text_softmax", ctypes.c_int), ("merge_mxfp8", ctypes.c_int)]


class CPrepParams(ctypes.Structure):
    _fields_ = [("grid_h", ctypes.c_int), ("grid_w", ctypes.c_int), ("kernel_h", ctypes.c_int),
                ("kernel_w", ctypes.c_int), ("taps", ctypes.c_int), ("causal", ctypes.c_int),
                ("l2_eps", ctypes.c_float)]


@dataclasses.dataclass(frozen=True)
class PrepParams:
    """VDA-Prep filter geometry (defaults: 3x3 spatial filter, 5 centred taps, eps 1e-6)."""
    grid_h: int
    grid_w: int
    kernel_h: int = 3
    kernel_w: int = 3
    taps: int = 5
    causal: int = 0
    l2_eps: float = 1e-6

    def c(self) -> CPrepParams:
        return CPrepParams(self.grid_h, self.grid_w, self.kernel_h, self.kernel_w, self.taps,
                           self.causal, self.l2_eps)


@dataclasses.dataclass(frozen=True)
class Params:
    """Operator hyper-parameters (defaults: 5-frame chunks, +-1 chunk window,
    anchors on, scale 1/sqrt(d_k) (0 = default), eps 1e-6, text split 1/2,
    text keys outside the Softmax branch, bf16 merge)."""
    softmax_scale: float = 0.0
    rms_eps: float = 1e-6
    text_init_scale: float = 0.5
    chunk_frames: int = 5
    window_chunks: int = 1
    anchors: int = 1
    text_softmax: int = 0
    merge_mxfp8: int = 0

    def c(self) -> CParams:
        return CParams(self.softmax_scale, self.rms_eps, self.text_init_scale,
                       self.chunk_frames, self.window_chunks, self.anchors, self.text_softmax,
                       self.merge_mxfp8)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with "
                           "`python -m softmax_attention_video_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dp, pp = ctypes.POINTER(Dims), ctypes.POINTER(CParams)
    L.vdn_default_params.argtypes = [pp]
    L.vdn_default_params.restype = None
    L.vdn_attn_fwd.argtypes = [P] * 17 + [S, dp, pp, I, P]
    L.vdn_attn_fwd.restype = I
    for n in ("vda_scan_fwd", "vda_scan_rev"):
        getattr(L, n).argtypes = [P] * 10 + [S, dp, pp, I, P]
        getattr(L, n).restype = I
    L.vdn_window_softmax_fwd.argtypes = [P] * 9 + [S, dp, pp, I, P]
    L.vdn_window_softmax_fwd.restype = I
    L.vdn_window_softmax_fwd_noalloc.argtypes = [P] * 8 + [dp, pp, I, P]
    L.vdn_window_softmax_fwd_noalloc.restype = I
    for n in ("vdn_workspace_bytes", "vdn_scan_workspace_bytes", "vdn_softmax_workspace_bytes",
              "vdn_merge_workspace_bytes"):
        getattr(L, n).argtypes = [dp, pp, I]
        getattr(L, n).restype = S
    L.vdn_window_plan.argtypes = [I, pp, P, P, P, P, P]
    L.vdn_window_plan.restype = I
    L.vdn_window_row_keys.argtypes = [dp, pp, I, P]
    L.vdn_window_row_keys.restype = I
    L.vdn_status_string.argtypes = [I]
    L.vdn_status_string.restype = ctypes.c_char_p
    L.vdn_last_error.argtypes = []
    L.vdn_last_error.restype = ctypes.c_char_p
    L.vdn_timer_enable.argtypes = [I]
    L.vdn_timer_enable.restype = I
    L.vdn_timer_read.argtypes = [P, I]
    L.vdn_timer_read.restype = I
    L.vdn_timer_disable.argtypes = []
    L.vdn_timer_disable.restype = None
    L.vda_prep_default_params.argtypes = [ctypes.POINTER(CPrepParams), I, I]
    L.vda_prep_default_params.restype = None
    L.vda_prep_fwd.argtypes = [P] * 8 + [dp, ctypes.POINTER(CPrepParams), I, P]
    L.vda_prep_fwd.restype = I
    L.vdn_merge_fwd.argtypes = [P] * 6 + [S, dp, pp, I, P]
    L.vdn_merge_fwd.restype = I
    L.vdn_mx_quantize.argtypes = [P, P, P, ctypes.c_longlong, I, P]
    L.vdn_mx_quantize.restype = I
    L.vdn_window_softmax_bwd.argtypes = [P] * 16 + [S, dp, pp, I, P]
    L.vdn_window_softmax_bwd.restype = I
    L.vdn_softmax_bwd_workspace_bytes.argtypes = [dp, pp, I]
    L.vdn_softmax_bwd_workspace_bytes.restype = S
    L.vdn_merge_bwd.argtypes = [P] * 10 + [S, dp, pp, I, P]
    L.vdn_merge_bwd.restype = I
    L.vdn_merge_bwd_workspace_bytes.argtypes = [dp, pp, I]
    L.vdn_merge_bwd_workspace_bytes.restype = S
    L.vda_bwd.argtypes = [P] * 22 + [S, dp, pp, I, P]
    L.vda_bwd.restype = I
    L.vda_bwd_workspace_bytes.argtypes = [dp, pp, I]
    L.vda_bwd_workspace_bytes.restype = S
    _lib = L
    return L


def _check(status: int):
    if status != VDN_OK:
        L = lib()
        raise VdnError(status, f"{L.vdn_status_string(status).decode()}: "
                               f"{L.vdn_last_error().decode()}")


def default_params() -> Params:
    c = CParams()
    lib().vdn_default_params(ctypes.byref(c))
    return Params(c.softmax_scale, c.rms_eps, c.text_init_scale, c.chunk_frames,
                  c.window_chunks, c.anchors, c.text_softmax, c.merge_mxfp8)


def window_plan(F: int, params: Params | None = None):
    """Host tables (vis [F,F] uint8, i_fwd, ws, i_rev, we [F] int32)."""
    p = (params or Params()).c()
    vis = np.zeros((F, F), np.uint8)
    t = [np.zeros(F, np.int32) for _ in range(4)]
    _check(lib().vdn_window_plan(F, ctypes.byref(p), vis.ctypes.data,
                                 *[a.ctypes.data for a in t]))
    return vis, *t


def window_row_keys(dims: Dims, params: Params | None = None, dtype: int = VDN_BF16):
    """Keys per query row of the forward Softmax launch ([B*H*L] int64; -1 =
    row not covered exactly once)."""
    p = (params or Params()).c()
    keys = np.zeros(dims.B * dims.H * dims.F * dims.N, np.int64)
    _check(lib().vdn_window_row_keys(ctypes.byref(dims), ctypes.byref(p), dtype, keys.ctypes.data))
    return keys


class KernelTimer:
    """Per-launch durations of the window Softmax kernel, from HIP events the
    library records around each launch on its stream (vdn_timer_*)."""

    def __init__(self, n: int):
        self.n = n
        _check(lib().vdn_timer_enable(n))

    def read(self) -> np.ndarray:
        ms = np.zeros(self.n, np.float32)
        k = lib().vdn_timer_read(ms.ctypes.data, self.n)
        if k < 0:
            _check(k)
        return ms[:k].astype(np.float64)

    def close(self):
        lib().vdn_timer_disable()


def workspace_bytes(dims: Dims, params: Params | None = None, dtype: int = VDN_BF16) -> int:
    p = (params or Params()).c()
    return int(lib().vdn_workspace_bytes(ctypes.byref(dims), ctypes.byref(p), dtype))


# ----------------------------------------------------------------------------
# torch-facing wrappers
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return VDN_BF16
    if t.dtype == torch.float32:
        return VDN_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t, name, dtype=None, shape=None, device=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    del torch
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


_WS_QUERY = {"attn": "vdn_workspace_bytes", "scan": "vdn_scan_workspace_bytes",
             "softmax": "vdn_softmax_workspace_bytes", "merge": "vdn_merge_workspace_bytes"}


def _workspace(dims, params, code, device, workspace, entry="attn"):
    """The caller's workspace, or a new one of the size the entry point needs."""
    torch = _torch()
    p = (params or Params()).c()
    need = int(getattr(lib(), _WS_QUERY[entry])(ctypes.byref(dims), ctypes.byref(p), code))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    if workspace.numel() < need:
        raise ValueError(f"workspace of {workspace.numel()} bytes < {need}")
    return workspace


def attn_fwd(q, k, v, beta, alpha, k_text, v_text, beta_text, g_s, g_l, gamma=None,
             W_s=None, W_l=None, out=None, ohat_s=None, ohat_l=None,
             params: Params | None = None, workspace=None, stream=None):
    """Full VDN attention forward (vdn_attn_fwd).

    q, k, v [B,H,L,d] (bf16 or fp32, frame-major); beta, g_s, g_l [B,H,L] fp32;
    alpha [B,H,F,d] fp32; k_text, v_text [B,H,T,d]; beta_text [B,H,T] fp32;
    gamma [d] fp32 or None; W_s, W_l [H*d, D] or None (identity).
    Returns out [B,L,D] (or [B,L,H*d] without projections).
    """
    torch = _torch()
    params = params or Params()
    B, H, L, d = q.shape
    F = alpha.shape[2]
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    N = L // F
    T = k_text.shape[2] if k_text is not None else 0
    dt = q.dtype
    code = _dtype_code(q)
    dev = q.device
    Dm = W_s.shape[1] if W_s is not None else H * d
    dims = Dims(B, H, F, N, T, d, d, Dm)
    f32 = torch.float32
    if out is None:
        out = torch.empty((B, L, Dm), dtype=dt, device=dev)
    ws = _workspace(dims, params, code, dev, workspace)
    p = params.c()
    args = [
        _ptr(q, "q", dt, (B, H, L, d), dev), _ptr(k, "k", dt, (B, H, L, d), dev),
        _ptr(v, "v", dt, (B, H, L, d), dev), _ptr(beta, "beta", f32, (B, H, L), dev),
        _ptr(alpha, "alpha", f32, (B, H, F, d), dev),
        _ptr(k_text, "k_text", dt, (B, H, T, d), dev, allow_none=T == 0),
        _ptr(v_text, "v_text", dt, (B, H, T, d), dev, allow_none=T == 0),
        _ptr(beta_text, "beta_text", f32, (B, H, T), dev, allow_none=T == 0),
        _ptr(g_s, "g_s", f32, (B, H, L), dev), _ptr(g_l, "g_l", f32, (B, H, L), dev),
        _ptr(gamma, "gamma", f32, (d,), dev, allow_none=True),
        _ptr(W_s, "W_s", dt, (H * d, Dm), dev, allow_none=True),
        _ptr(W_l, "W_l", dt, (H * d, Dm), dev, allow_none=True),
        _ptr(out, "out", dt, (B, L, Dm), dev),
        _ptr(ohat_s, "ohat_s", dt, (B, L, H, d), dev, allow_none=True),
        _ptr(ohat_l, "ohat_l", dt, (B, L, H, d), dev, allow_none=True),
        ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
    ]
    _check(lib().vdn_attn_fwd(*args, ctypes.byref(dims), ctypes.byref(p), code,
                              _stream(stream, dev)))
    return out


def _scan(which, k, v, beta, alpha, k_text, v_text, beta_text, params, workspace, stream,
          P=None, S_text=None):
    torch = _torch()
    params = params or Params()
    B, H, L, d = k.shape
    F = alpha.shape[2]
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    N = L // F
    T = k_text.shape[2] if k_text is not None else 0
    dt = k.dtype
    code = _dtype_code(k)
    dev = k.device
    C = F // params.chunk_frames
    dims = Dims(B, H, F, N, T, d, d, H * d)
    f32 = torch.float32
    if P is None:
        P = torch.empty((B, H, C + 1, d, d), dtype=f32, device=dev)
    if S_text is None:
        S_text = torch.empty((B, H, d, d), dtype=f32, device=dev)
    ws = _workspace(dims, params, code, dev, workspace, "scan")
    p = params.c()
    fn = lib().vda_scan_fwd if which == "fwd" else lib().vda_scan_rev
    _check(fn(_ptr(k, "k", dt, (B, H, L, d), dev), _ptr(v, "v", dt, (B, H, L, d), dev),
              _ptr(beta, "beta", f32, (B, H, L), dev), _ptr(alpha, "alpha", f32, (B, H, F, d), dev),
              _ptr(k_text, "k_text", dt, (B, H, T, d), dev, allow_none=T == 0),
              _ptr(v_text, "v_text", dt, (B, H, T, d), dev, allow_none=T == 0),
              _ptr(beta_text, "beta_text", f32, (B, H, T), dev, allow_none=T == 0),
              _ptr(P, "P", f32, (B, H, C + 1, d, d), dev),
              _ptr(S_text, "S_text", f32, (B, H, d, d), dev),
              ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
              ctypes.byref(dims), ctypes.byref(p), code, _stream(stream, dev)))
    return P, S_text


def scan_fwd(k, v, beta, alpha, k_text, v_text, beta_text, params=None, workspace=None,
             stream=None, P=None, S_text=None):
    """Forward VDA chunk-boundary states P_fwd [B,H,C+1,d,d] and S_text (vda_scan_fwd)."""
    return _scan("fwd", k, v, beta, alpha, k_text, v_text, beta_text, params, workspace,
                 stream, P, S_text)


def scan_rev(k, v, beta, alpha, k_text, v_text, beta_text, params=None, workspace=None,
             stream=None, P=None, S_text=None):
    """Reverse VDA chunk-boundary states P_rev [B,H,C+1,d,d] and S_text (vda_scan_rev)."""
    return _scan("rev", k, v, beta, alpha, k_text, v_text, beta_text, params, workspace,
                 stream, P, S_text)


def window_softmax_fwd(q, k, v, F: int, g_s=None, want_lse: bool = False, out=None,
                       params: Params | None = None, workspace=None, stream=None,
                       k_text=None, v_text=None):
    """Window/anchor Softmax branch (vdn_window_softmax_fwd).  With
    params.text_softmax the text keys k_text, v_text [B,H,T,d] join every
    query's keys.  Returns (out [B,L,H,d], lse [B,H,L] or None)."""
    torch = _torch()
    params = params or Params()
    B, H, L, d = q.shape
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    N = L // F
    dt = q.dtype
    code = _dtype_code(q)
    dev = q.device
    T = k_text.shape[2] if k_text is not None else 0
    dims = Dims(B, H, F, N, T, d, d, H * d)
    if out is None:
        out = torch.empty((B, L, H, d), dtype=dt, device=dev)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=dev) if want_lse else None
    ws = _workspace(dims, params, code, dev, workspace, "softmax")
    p = params.c()
    _check(lib().vdn_window_softmax_fwd(
        _ptr(q, "q", dt, (B, H, L, d), dev), _ptr(k, "k", dt, (B, H, L, d), dev),
        _ptr(v, "v", dt, (B, H, L, d), dev),
        _ptr(k_text, "k_text", dt, (B, H, T, d), dev, allow_none=True),
        _ptr(v_text, "v_text", dt, (B, H, T, d), dev, allow_none=T == 0),
        _ptr(g_s, "g_s", torch.float32, (B, H, L), dev, allow_none=True),
        _ptr(out, "out", dt, (B, L, H, d), dev),
        _ptr(lse, "lse", torch.float32, (B, H, L), dev, allow_none=True),
        ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
        ctypes.byref(dims), ctypes.byref(p), code, _stream(stream, dev)))
    return out, lse


def window_softmax_fwd_noalloc(q, k, v, F: int, out, lse=None, g_s=None,
                               params: Params | None = None, stream=None, k_text=None,
                               v_text=None):
    """vdn_window_softmax_fwd_noalloc: the Softmax branch with the library's
    own device scratch.  The caller supplies out [B,L,H,d] (and optionally
    lse [B,H,L]); nothing is allocated here or in the library."""
    torch = _torch()
    params = params or Params()
    B, H, L, d = q.shape
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    dt = q.dtype
    dev = q.device
    T = k_text.shape[2] if k_text is not None else 0
    dims = Dims(B, H, F, L // F, T, d, d, H * d)
    p = params.c()
    _check(lib().vdn_window_softmax_fwd_noalloc(
        _ptr(q, "q", dt, (B, H, L, d), dev), _ptr(k, "k", dt, (B, H, L, d), dev),
        _ptr(v, "v", dt, (B, H, L, d), dev),
        _ptr(k_text, "k_text", dt, (B, H, T, d), dev, allow_none=True),
        _ptr(v_text, "v_text", dt, (B, H, T, d), dev, allow_none=T == 0),
        _ptr(g_s, "g_s", torch.float32, (B, H, L), dev, allow_none=True),
        _ptr(out, "out", dt, (B, L, H, d), dev),
        _ptr(lse, "lse", torch.float32, (B, H, L), dev, allow_none=True),
        ctypes.byref(dims), ctypes.byref(p), _dtype_code(q), _stream(stream, dev)))
    return out, lse


def window_softmax_bwd(q, k, v, o, lse, d_out, F: int, g_s=None, want_dg: bool = False,
                       params: Params | None = None, workspace=None, stream=None, k_text=None,
                       v_text=None):
    """Gradients of the Softmax branch (vdn_window_softmax_bwd).

    q, k, v [B,H,L,d]; o [B,L,H,d] the ungated output and lse [B,H,L] of
    window_softmax_fwd(..., g_s=None, want_lse=True) with the same params
    and text keys; d_out [B,L,H,d] the gradient of the gated output; g_s
    [B,H,L] or None.  With params.text_softmax, k_text and v_text [B,H,T,d]
    are keys of every query.  Returns (dq, dk, dv [B,H,L,d], dg [B,H,L] or
    None), followed by (dk_text, dv_text [B,H,T,d]) with text keys."""
    torch = _torch()
    params = params or Params()
    B, H, L, d = q.shape
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    dt = q.dtype
    code = _dtype_code(q)
    dev = q.device
    f32 = torch.float32
    T = k_text.shape[2] if k_text is not None else 0
    text = bool(params.text_softmax) and T > 0
    dims = Dims(B, H, F, L // F, T, d, d, H * d)
    p = params.c()
    need = int(lib().vdn_softmax_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(p), code))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() < need:
        raise ValueError(f"workspace of {workspace.numel()} bytes < {need}")
    dq, dk, dv = (torch.empty((B, H, L, d), dtype=dt, device=dev) for _ in range(3))
    dg = torch.empty((B, H, L), dtype=f32, device=dev) if want_dg else None
    dkt, dvt = ((torch.empty((B, H, T, d), dtype=dt, device=dev) for _ in range(2)) if text
                else (None, None))
    _check(lib().vdn_window_softmax_bwd(
        _ptr(q, "q", dt, (B, H, L, d), dev), _ptr(k, "k", dt, (B, H, L, d), dev),
        _ptr(v, "v", dt, (B, H, L, d), dev),
        _ptr(k_text if text else None, "k_text", dt, (B, H, T, d), dev, allow_none=True),
        _ptr(v_text if text else None, "v_text", dt, (B, H, T, d), dev, allow_none=True),
        _ptr(o, "o", dt, (B, L, H, d), dev),
        _ptr(lse, "lse", f32, (B, H, L), dev), _ptr(g_s, "g_s", f32, (B, H, L), dev, allow_none=True),
        _ptr(d_out, "d_out", dt, (B, L, H, d), dev), _ptr(dq, "dq"), _ptr(dk, "dk"), _ptr(dv, "dv"),
        _ptr(dkt, "dk_text", allow_none=True), _ptr(dvt, "dv_text", allow_none=True),
        _ptr(dg, "dg", allow_none=True),
        ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
        ctypes.byref(dims), ctypes.byref(p), code, _stream(stream, dev)))
    if text:
        return dq, dk, dv, dg, dkt, dvt
    return dq, dk, dv, dg


def vda_bwd(q, k, v, beta, alpha, k_text, v_text, beta_text, g_l, d_out, gamma=None,
            want_dg: bool = False, want_dgamma: bool = False, params: Params | None = None,
            workspace=None, stream=None):
    """Gradients of the linear (VDA) branch output Ohat_l (vda_bwd).

    Inputs as for attn_fwd (q, k, v [B,H,L,d]; beta, g_l [B,H,L]; alpha
    [B,H,F,d]; k_text, v_text [B,H,T,d]; beta_text [B,H,T]; gamma [d] or
    None); d_out [B,L,H,d] the gradient of Ohat_l.  Returns a dict with dq,
    dk, dv [B,H,L,d]; dbeta [B,H,L]; dalpha [B,H,F,d]; dk_text, dv_text
    [B,H,T,d]; dbeta_text [B,H,T]; dg_l [B,H,L] and dgamma [d] when asked."""
    torch = _torch()
    params = params or Params()
    B, H, L, d = q.shape
    F = alpha.shape[2]
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    T = k_text.shape[2]
    dt = q.dtype
    code = _dtype_code(q)
    dev = q.device
    f32 = torch.float32
    dims = Dims(B, H, F, L // F, T, d, d, H * d)
    p = params.c()
    need = int(lib().vda_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(p), code))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() < need:
        raise ValueError(f"workspace of {workspace.numel()} bytes < {need}")
    out = dict(dq=torch.empty((B, H, L, d), dtype=dt, device=dev),
               dk=torch.empty((B, H, L, d), dtype=dt, device=dev),
               dv=torch.empty((B, H, L, d), dtype=dt, device=dev),
               dbeta=torch.empty((B, H, L), dtype=f32, device=dev),
               dalpha=torch.empty((B, H, F, d), dtype=f32, device=dev),
               dk_text=torch.empty((B, H, T, d), dtype=dt, device=dev),
               dv_text=torch.empty((B, H, T, d), dtype=dt, device=dev),
               dbeta_text=torch.empty((B, H, T), dtype=f32, device=dev),
               dg_l=torch.empty((B, H, L), dtype=f32, device=dev) if want_dg else None,
               dgamma=torch.empty((d,), dtype=f32, device=dev) if want_dgamma else None)
    tx = T > 0
    _check(lib().vda_bwd(
        _ptr(q, "q", dt, (B, H, L, d), dev), _ptr(k, "k", dt, (B, H, L, d), dev),
        _ptr(v, "v", dt, (B, H, L, d), dev), _ptr(beta, "beta", f32, (B, H, L), dev),
        _ptr(alpha, "alpha", f32, (B, H, F, d), dev),
        _ptr(k_text if tx else None, "k_text", dt, (B, H, T, d), dev, allow_none=True),
        _ptr(v_text if tx else None, "v_text", dt, (B, H, T, d), dev, allow_none=True),
        _ptr(beta_text if tx else None, "beta_text", f32, (B, H, T), dev, allow_none=True),
        _ptr(g_l, "g_l", f32, (B, H, L), dev),
        _ptr(gamma, "gamma", f32, (d,), dev, allow_none=True),
        _ptr(d_out, "d_out", dt, (B, L, H, d), dev),
        _ptr(out["dq"], "dq"), _ptr(out["dk"], "dk"), _ptr(out["dv"], "dv"),
        _ptr(out["dbeta"], "dbeta"), _ptr(out["dalpha"], "dalpha"),
        _ptr(out["dk_text"] if tx else None, "dk_text", allow_none=True),
        _ptr(out["dv_text"] if tx else None, "dv_text", allow_none=True),
        _ptr(out["dbeta_text"] if tx else None, "dbeta_text", allow_none=True),
        _ptr(out["dg_l"], "dg_l", allow_none=True), _ptr(out["dgamma"], "dgamma", allow_none=True),
        ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
        ctypes.byref(dims), ctypes.byref(p), code, _stream(stream, dev)))
    return out


def merge_fwd(ohat_s, ohat_l, W_s, W_l, F: int, params: Params | None = None, out=None,
              workspace=None, stream=None):
    """The merge alone (vdn_merge_fwd): out [B,L,D] = Ohat_s W_s + Ohat_l W_l
    (bf16, or MX-FP8 with params.merge_mxfp8).  ohat_* [B,L,H,d]; W_* [H*d, D]
    or both None (identity, D = H*d)."""
    torch = _torch()
    params = params or Params()
    B, L, H, d = ohat_s.shape
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    dt = ohat_s.dtype
    code = _dtype_code(ohat_s)
    dev = ohat_s.device
    Dm = W_s.shape[1] if W_s is not None else H * d
    dims = Dims(B, H, F, L // F, 0, d, d, Dm)
    if out is None:
        out = torch.empty((B, L, Dm), dtype=dt, device=dev)
    ws = _workspace(dims, params, code, dev, workspace, "merge")
    p = params.c()
    _check(lib().vdn_merge_fwd(
        _ptr(ohat_s, "ohat_s", dt, (B, L, H, d), dev), _ptr(ohat_l, "ohat_l", dt, (B, L, H, d), dev),
        _ptr(W_s, "W_s", dt, (H * d, Dm), dev, allow_none=True),
        _ptr(W_l, "W_l", dt, (H * d, Dm), dev, allow_none=True),
        _ptr(out, "out", dt, (B, L, Dm), dev),
        ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()),
        ctypes.byref(dims), ctypes.byref(p), code, _stream(stream, dev)))
    return out



def merge_bwd(d_out, ohat_s, ohat_l, W_s, W_l, F: int, want_dw: bool = True,
              params: Params | None = None, workspace=None, stream=None):
    """Gradients of the merge (vdn_merge_bwd).  d_out [B,L,D]; ohat_* [B,L,H,d];
    W_* [H*d, D] or both None (identity).  Returns (d_ohat_s, d_ohat_l
    [B,L,H,d], dW_s, dW_l [H*d, D] or None)."""
    torch = _torch()
    params = params or Params()
    B, L, H, d = ohat_s.shape
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    dt = ohat_s.dtype
    code = _dtype_code(ohat_s)
    dev = ohat_s.device
    Dm = W_s.shape[1] if W_s is not None else H * d
    dims = Dims(B, H, F, L // F, 0, d, d, Dm)
    p = params.c()
    want_dw = want_dw and W_s is not None
    need = int(lib().vdn_merge_bwd_workspace_bytes(ctypes.byref(dims), ctypes.byref(p), code)) if want_dw else 0
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.numel() < need:
        raise ValueError(f"workspace of {workspace.numel()} bytes < {need}")
    dos, dol = (torch.empty((B, L, H, d), dtype=dt, device=dev) for _ in range(2))
    dws, dwl = ((torch.empty((H * d, Dm), dtype=dt, device=dev) for _ in range(2)) if want_dw
                else (None, None))
    _check(lib().vdn_merge_bwd(
        _ptr(ohat_s, "ohat_s", dt, (B, L, H, d), dev), _ptr(ohat_l, "ohat_l", dt, (B, L, H, d), dev),
        _ptr(W_s, "W_s", dt, (H * d, Dm), dev, allow_none=True),
        _ptr(W_l, "W_l", dt, (H * d, Dm), dev, allow_none=True),
        _ptr(d_out, "d_out", dt, (B, L, Dm), dev), _ptr(dos, "d_ohat_s"), _ptr(dol, "d_ohat_l"),
        _ptr(dws, "dW_s", allow_none=True), _ptr(dwl, "dW_l", allow_none=True),
        ctypes.c_void_p(workspace.data_ptr()), ctypes.c_size_t(workspace.numel()),
        ctypes.byref(dims), ctypes.byref(p), code, _stream(stream, dev)))
    return dos, dol, dws, dwl


def mx_quantize(x, stream=None):
    """MX-FP8 of a bf16 matrix [rows, cols] along its rows (vdn_mx_quantize).
    Returns (codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [rows, cols]")
    rows, cols = x.shape
    dev = x.device
    if cols % 32:
        raise ValueError(f"cols={cols} is not a multiple of 32")
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    if rows == 0 or cols == 0:
        return codes, scales
    _check(lib().vdn_mx_quantize(_ptr(x, "x", torch.bfloat16, (rows, cols), dev),
                                 _ptr(codes, "codes"), _ptr(scales, "scales"),
                                 ctypes.c_longlong(rows), ctypes.c_int(cols), _stream(stream, dev)))
    return codes, scales


def prep_fwd(q, k, v, w_spatial, w_temporal, F: int, params: PrepParams, q_out=None, k_out=None,
             v_out=None, stream=None):
    """VDA-Prep, the linear branch's feature map (vda_prep_fwd).

    q, k, v [B,L,H,d] token-major (bf16 or fp32); w_spatial [H,d,kh,kw] and
    w_temporal [H,d,taps] fp32.  Returns (q', k', v'), each [B,H,L,d]."""
    torch = _torch()
    B, L, H, d = q.shape
    if L % F:
        raise ValueError(f"L={L} is not a multiple of F={F}")
    N = L // F
    dt = q.dtype
    code = _dtype_code(q)
    dev = q.device
    dims = Dims(B, H, F, N, 0, d, d, H * d)
    outs = []
    for o in (q_out, k_out, v_out):
        outs.append(o if o is not None else torch.empty((B, H, L, d), dtype=dt, device=dev))
    p = params.c()
    _check(lib().vda_prep_fwd(
        _ptr(q, "q", dt, (B, L, H, d), dev), _ptr(k, "k", dt, (B, L, H, d), dev),
        _ptr(v, "v", dt, (B, L, H, d), dev),
        _ptr(w_spatial, "w_spatial", torch.float32, (H, d, params.kernel_h, params.kernel_w), dev),
        _ptr(w_temporal, "w_temporal", torch.float32, (H, d, params.taps), dev),
        _ptr(outs[0], "q_out", dt, (B, H, L, d), dev), _ptr(outs[1], "k_out", dt, (B, H, L, d), dev),
        _ptr(outs[2], "v_out", dt, (B, H, L, d), dev),
        ctypes.byref(dims), ctypes.byref(p), code, _stream(stream, dev)))
    return tuple(outs)
