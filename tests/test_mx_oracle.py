"""Pins of the MX-FP8 oracle (OCP Microscaling v1.0, E4M3 elements, blocks
of 32) to what the format definition and a library routine fix: torch's own
float8_e4m3fn conversions (decode of every byte, round-to-nearest-even
encode in range), the saturation rule, the shared-exponent rule, exact round
trips of representable blocks, the element error bound, and a brute-force
product."""
import numpy as np
import pytest
import torch

from oracle import mx_merge as MX


def test_decode_every_byte_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = MX.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    # landmarks of the format
    assert MX.e4m3_decode([0x7E])[0] == 448.0 and MX.e4m3_decode([0x08])[0] == 2.0 ** -6
    assert MX.e4m3_decode([0x01])[0] == 2.0 ** -9 and np.isnan(MX.e4m3_decode([0x7F])[0])


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    np.testing.assert_array_equal(MX.e4m3_encode(MX.e4m3_decode(codes)), codes)


def test_encode_matches_torch_in_range_including_ties():
    rng = np.random.default_rng(0)
    vals = [rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 2.0 ** rng.integers(-12, 8, 4000)]
    # exact midpoints between neighbouring representables (ties go to the even code)
    pos = MX.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[1:] + pos[:-1]) / 2
    m32 = mids.astype(np.float32)      # midpoints are exact in fp32; so are their fp32 neighbours
    vals += [m32, -m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))]
    # fp32 inputs, so that torch's conversion rounds once (as the oracle does)
    x = np.concatenate([np.asarray(v, np.float64).astype(np.float32) for v in vals])
    x = x[np.abs(x) < 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = MX.e4m3_encode(x.astype(np.float64))
    # torch keeps the sign of values that round to zero, as the oracle does
    np.testing.assert_array_equal(got, want)


def test_encode_saturates_above_max():
    x = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 511.9, 1e6, -470.0, -1e30])
    got = MX.e4m3_encode(x)
    np.testing.assert_array_equal(got, [0x7E] * 7 + [0xFE, 0xFE])


def test_shared_exponent_rule():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200, 64)) * np.exp2(rng.integers(-30, 30, (200, 1)))
    codes, scales = MX.mx_quantize(x)
    s = scales.astype(np.int64) - 127
    amax = np.abs(x.reshape(200, 2, 32)).max(axis=-1)
    r = amax / np.exp2(s)
    assert np.all((r >= 256) & (r < 512))
    # the largest element of a block lands in the top binade (or saturates)
    top = np.abs(MX.e4m3_decode(codes).reshape(200, 2, 32)).max(axis=-1)
    assert np.all(top >= 256)


def test_zero_and_tiny_blocks():
    codes, scales = MX.mx_quantize(np.zeros((2, 32)))
    assert not codes.any() and not scales.any()
    # a block of the smallest bf16 subnormals clamps the scale at 2^-127
    tiny = np.full((1, 32), 2.0 ** -133)
    codes, scales = MX.mx_quantize(tiny)
    assert scales[0, 0] == 0
    np.testing.assert_array_equal(MX.mx_dequantize(codes, scales), tiny)


def test_representable_blocks_round_trip_exactly():
    rng = np.random.default_rng(2)
    pos = MX.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    blocks = rng.choice(pos, size=(50, 32)) * rng.choice([-1.0, 1.0], size=(50, 32))
    blocks[:, 0] = rng.choice(pos[pos >= 256], size=50)      # each block reaches the top binade
    e = rng.integers(-40, 40, size=(50, 1))
    x = blocks * np.exp2(e)
    codes, scales = MX.mx_quantize(x)
    np.testing.assert_array_equal(MX.mx_dequantize(codes, scales), x)


def test_element_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 32)) * np.exp2(rng.integers(-8, 8, (300, 1)))
    codes, scales = MX.mx_quantize(x)
    y = MX.mx_dequantize(codes, scales)
    X = np.exp2(scales.astype(np.float64) - 127)[:, :1]
    u = np.abs(x) / X                                       # element magnitude in scale units
    binade = np.floor(np.log2(np.maximum(u, 2.0 ** -6)))
    half_ulp = np.where(u >= 448, 64.0, np.exp2(binade - 4))  # half of 2^(binade - 3)
    assert np.all(np.abs(y - x) <= half_ulp * X * (1 + 1e-12))


def test_mx_merge_equals_brute_force_on_dequantized_operands():
    rng = np.random.default_rng(4)
    B, L, H, dv, D = 1, 5, 2, 32, 7
    os_, ol = rng.standard_normal((B, L, H, dv)), rng.standard_normal((B, L, H, dv))
    ws, wl = rng.standard_normal((H * dv, D)) * 0.1, rng.standard_normal((H * dv, D)) * 0.1
    out, q = MX.mx_merge(os_, ol, ws, wl)
    A = MX.mx_dequantize(q["a_codes"], q["a_scales"])
    Wt = MX.mx_dequantize(q["w_codes"], q["w_scales"])
    K2 = 2 * H * dv
    for m in range(B * L):
        for n in range(D):
            s = 0.0
            for k in range(K2):
                s += A[m, k] * Wt[n, k]
            assert abs(out.reshape(B * L, D)[m, n] - s) <= 1e-12 * max(1.0, abs(s))
    # the quantized operands are the blocks of [Ohat_s | Ohat_l] and of [W_s ; W_l]^T
    ca, _ = MX.mx_quantize(os_.reshape(B * L, H * dv))
    np.testing.assert_array_equal(q["a_codes"][:, :H * dv], ca)
    cw, _ = MX.mx_quantize(wl.T)
    np.testing.assert_array_equal(q["w_codes"][:, H * dv:], cw)


def test_mx_merge_close_to_exact_merge():
    rng = np.random.default_rng(5)
    B, L, H, dv, D = 1, 64, 4, 64, 48
    os_, ol = rng.standard_normal((B, L, H, dv)), rng.standard_normal((B, L, H, dv))
    ws, wl = rng.standard_normal((H * dv, D)) * 0.05, rng.standard_normal((H * dv, D)) * 0.05
    out, _ = MX.mx_merge(os_, ol, ws, wl)
    exact = os_.reshape(B, L, -1) @ ws + ol.reshape(B, L, -1) @ wl
    rel = np.linalg.norm(out - exact) / np.linalg.norm(exact)
    assert 1e-3 < rel < 0.08, rel


def test_rejects_bad_block_length():
    with pytest.raises(ValueError):
        MX.mx_quantize(np.ones((2, 48)))
