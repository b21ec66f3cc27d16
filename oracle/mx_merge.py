"""MX-FP8 merge projections -- CPU fp64 oracle.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and shares no code with it.

Source: "Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
Generation" (arXiv 2609.20744), system section, other optimizations: the
wide output GEMMs run in MXFP8 while recurrent states and the small-matrix
inverses stay in FP32.  Here that is the merge of the two branches,
out = [Ohat_s | Ohat_l] [W_s ; W_l], with both operands in MX-FP8.

The format is the published OCP Microscaling (MX) v1.0 definition:
  * a block of 32 consecutive elements shares one scale X = 2^s stored as an
    E8M0 byte (s + 127);
  * s = floor(log2(max |v|)) - 8, where 8 is the largest exponent of the
    element format, clamped to the E8M0 range [-127, 127];
  * each element is v / X converted to FP8 E4M3 (sign, 4 exponent bits with
    bias 7, 3 mantissa bits; subnormals; no infinities; S.1111.111 is NaN;
    largest finite 448) by round-to-nearest-even, values beyond 448 clamped
    to 448 (saturation).

Readings where the page is silent (each also listed in the design notes):
  * element format E4M3 (the page says MXFP8 only);
  * blocks run along the contraction index for both operands: along
    K = H*d_v within each of Ohat_s and Ohat_l (K a multiple of 32), and
    down each column of W_s and W_l;
  * a block of zeros gets scale byte 0 (2^-127) and zero codes; the sign of
    a value that rounds to zero is kept in the code;
  * the product is exact in fp64 of the dequantized operands (the hardware
    accumulates in fp32); the output is then stored like the bf16 merge.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
EMAX_E4M3 = 8
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 byte (NaN for S.1111.111)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# every finite non-negative E4M3 value, ascending, with its code
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code, magnitudes
    above 448 saturate to 448; the sign bit is the sign of x)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    if np.isnan(a).any():
        raise ValueError("NaN input")
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = np.abs(_POS_VALUES[hi] - a)
    d_lo = np.abs(a - _POS_VALUES[lo])
    take_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (_POS_CODES[lo] % 2 == 0))
    code = np.where(take_lo, _POS_CODES[lo], _POS_CODES[hi]).astype(np.uint8)
    code = np.where(a >= E4M3_MAX, np.uint8(0x7E), code)
    neg = np.signbit(x)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def mx_scale_exponent(amax) -> np.ndarray:
    """Shared exponent s of blocks with the given max magnitude."""
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(amax)          # amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1
    s = (e - 1) - EMAX_E4M3
    s = np.where(amax > 0, s, -127)
    return np.clip(s, -127, 127).astype(np.int64)


def mx_quantize(x):
    """MX-FP8 of x along its last axis (length a multiple of 32).

    Returns (codes uint8, same shape as x; scale bytes uint8, shape
    x.shape[:-1] + (n / 32,))."""
    x = np.asarray(x, np.float64)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError(f"last axis {n} is not a multiple of {BLOCK}")
    xb = x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))
    s = mx_scale_exponent(np.abs(xb).max(axis=-1))
    codes = e4m3_encode(xb / np.exp2(s)[..., None])
    return codes.reshape(x.shape), (s + 127).astype(np.uint8)


def mx_dequantize(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, np.uint8)
    n = codes.shape[-1]
    v = e4m3_decode(codes).reshape(codes.shape[:-1] + (n // BLOCK, BLOCK))
    x = np.exp2(np.asarray(scales, np.float64) - 127.0)[..., None]
    return (v * x).reshape(codes.shape)


def mx_merge(Ohat_s, Ohat_l, W_s, W_l):
    """out = deq(MX(A)) deq(MX(W)) with A = [Ohat_s | Ohat_l] over the heads
    and W = [W_s ; W_l]; blocks of 32 along the contraction index.

    Ohat_*: [B, L, H, dv]; W_*: [H*dv, D].  Returns (out [B, L, D], and the
    quantized operands as a dict: A codes / scales [B*L, 2K], W^T codes /
    scales [D, 2K])."""
    Ohat_s = np.asarray(Ohat_s, np.float64)
    B, L, H, dv = Ohat_s.shape
    K = H * dv
    A = np.concatenate([Ohat_s.reshape(B * L, K), np.asarray(Ohat_l, np.float64).reshape(B * L, K)],
                       axis=1)
    Wt = np.concatenate([np.asarray(W_s, np.float64), np.asarray(W_l, np.float64)], axis=0).T
    ca, sa = mx_quantize(A)
    cw, sw = mx_quantize(Wt)
    out = mx_dequantize(ca, sa) @ mx_dequantize(cw, sw).T
    D = Wt.shape[0]
    return out.reshape(B, L, D), {"a_codes": ca, "a_scales": sa, "w_codes": cw, "w_scales": sw}
