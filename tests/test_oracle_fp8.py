"""Pins of the MXFP8 oracle (oracle/fp8.py) to facts other than itself.

The E4M3 decoder is pinned to values fixed by the format (bias 7, 3 mantissa
bits, subnormals m * 2^-9, largest finite 448, NaN codes); the encoder to a
brute-force nearest-value search with ties to even, to saturation, and to
the round trip over every code; the block scale to its closed form; the
quantizer to its error bounds and layout; MXFP8 attention to attention on
the dequantized inputs; the P-rounding bound to a simulation of the
rounding it bounds. Planted mistakes at the end must fail a pin.
"""

import math

import numpy as np
import pytest

from oracle import (
    attention_forward,
    attention_forward_mxfp8,
    e4m3_decode,
    e4m3_encode,
    mx_dequantize,
    mx_quantize,
    mx_scale_code,
    p_rounding_bound,
)


def test_decode_fixed_values():
    assert e4m3_decode(0x7E) == 448.0
    assert e4m3_decode(0x01) == 2.0 ** -9
    assert e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert e4m3_decode(0x08) == 2.0 ** -6
    assert e4m3_decode(0x38) == 1.0
    assert e4m3_decode(0x40) == 2.0
    assert e4m3_decode(0x3C) == 1.5
    assert e4m3_decode(0xB8) == -1.0
    assert e4m3_decode(0x78) == 256.0
    assert math.isnan(e4m3_decode(0x7F)) and math.isnan(e4m3_decode(0xFF))
    z = e4m3_decode(0x80)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    vals = e4m3_decode(np.arange(256))
    assert np.isnan(vals).sum() == 2
    mags = e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(mags) > 0)  # codes 0x00 .. 0x7e increase strictly


def test_round_trip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def _brute_encode(x):
    mags = [float(e4m3_decode(c)) for c in range(0x7F)]
    a = min(abs(x), 448.0)
    best = min(range(len(mags)), key=lambda c: (abs(mags[c] - a), c & 1))  # ties: even code
    return best | (0x80 if (x < 0 or (x == 0 and math.copysign(1, x) < 0)) else 0)


def test_encode_matches_brute_force_nearest_ties_even():
    rng = np.random.default_rng(1)
    mags = e4m3_decode(np.arange(0x7F))
    mids = (mags[1:] + mags[:-1]) / 2  # every tie
    xs = np.concatenate([rng.standard_normal(300) * 30, rng.standard_normal(100) * 1e-2, mids, -mids,
                         [0.0, 1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, 3 * 2.0 ** -10]])
    got = e4m3_encode(xs)
    want = np.array([_brute_encode(float(x)) for x in xs], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)
    assert e4m3_encode(1.0625) == 0x38 and e4m3_encode(1.1875) == 0x3A  # ties go to the even mantissa
    assert e4m3_encode(2.0 ** -10) == 0x00 and e4m3_encode(3 * 2.0 ** -10) == 0x02


def test_encode_saturates():
    np.testing.assert_array_equal(e4m3_encode([449.0, 464.0, 480.0, 1e9, -1e9]),
                                  np.array([0x7E, 0x7E, 0x7E, 0x7E, 0xFE], dtype=np.uint8))
    with pytest.raises(ValueError):
        e4m3_encode([np.nan])


def test_scale_code_closed_forms():
    # smallest 2^e with amax <= 448 * 2^e, biased by 127
    amax = [1.0, 448.0, 449.0, 256.0, 255.9, 224.0, 224.1, 0.0, 2.0 ** -130, 3.0, 3.5, 3.6]
    want = [119, 127, 128, 127, 127, 126, 127, 0, 0, 120, 120, 121]
    np.testing.assert_array_equal(mx_scale_code(amax), np.array(want, dtype=np.uint8))
    for a, c in zip(amax, want):  # the definition, checked directly
        if a > 0 and 0 < c < 254:
            assert a <= 448 * 2.0 ** (c - 127) and a > 448 * 2.0 ** (c - 128)


def test_quantize_constant_block_and_layout():
    x = np.ones((2, 64))
    c, s = mx_quantize(x)
    assert c.shape == (2, 64) and s.shape == (2, 2)
    assert np.all(c == 0x78) and np.all(s == 119)  # 1 = 256 * 2^-8
    ct, st = mx_quantize(x.T, axis=0)  # blocks along the other axis of the transpose
    np.testing.assert_array_equal(ct, c.T)
    np.testing.assert_array_equal(st, s.T)
    with pytest.raises(ValueError):
        mx_quantize(np.ones((2, 40)))


@pytest.mark.parametrize("std", [1.0, 1e-3, 300.0])
def test_quantize_error_bounds(std):
    rng = np.random.default_rng(int(std * 10) + 3)
    x = rng.standard_normal((16, 128)) * std
    c, s = mx_quantize(x)
    xh = mx_dequantize(c, s)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127.0), 32, axis=-1)
    amax = np.repeat(np.abs(x).reshape(16, 4, 32).max(-1), 32, axis=-1)
    # the block maximum lands in [224, 448] after scaling (nothing saturates)
    top = np.abs(e4m3_decode(c)).reshape(16, 4, 32).max(-1)
    assert np.all(top >= 224) and np.all(top <= 448)
    err = np.abs(xh - x)
    normal = np.abs(x) / scale >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]))
    assert np.all(err[~normal] <= 2.0 ** -10 * scale[~normal])
    assert np.all(err <= 2.0 ** -4 * amax)


def test_mxfp8_attention_is_attention_on_dequantized_inputs():
    rng = np.random.default_rng(7)
    n, d = 64, 64
    q, k, v = (rng.standard_normal((2, n, d)) for _ in range(3))
    q8, qs = mx_quantize(q)
    k8, ks = mx_quantize(k)
    vt8, vts = mx_quantize(np.swapaxes(v, -1, -2))  # V^T [d, n], blocks along the keys
    o, lse = attention_forward_mxfp8(q8, qs, k8, ks, vt8, vts, 0.125)
    qh, kh = mx_dequantize(q8, qs), mx_dequantize(k8, ks)
    vh = np.swapaxes(mx_dequantize(vt8, vts), -1, -2)
    o2, l2 = attention_forward(qh, kh, vh, 0.125)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)
    # inputs that are exact in MXFP8 (values from a set every block scale keeps exact)
    pick = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -1.5, 2.0, -2.0, 3.0, -3.0])
    qi, ki, vi = (pick[rng.integers(0, len(pick), (2, n, d))] for _ in range(3))
    qi8, qis = mx_quantize(qi)
    ki8, kis = mx_quantize(ki)
    vi8, vis = mx_quantize(np.swapaxes(vi, -1, -2))
    oe, le = attention_forward_mxfp8(qi8, qis, ki8, kis, vi8, vis, 0.125)
    o3, l3 = attention_forward(qi, ki, vi, 0.125)
    np.testing.assert_allclose(oe, o3, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(le, l3, rtol=1e-13, atol=1e-14)


def test_p_rounding_bound_holds_for_simulated_rounding():
    # Round every P_ij to E4M3 after an arbitrary power-of-two block scale (any
    # scale that keeps the block in E4M3's normal range gives the same
    # relative rounding) and check |delta O| against the bound.
    rng = np.random.default_rng(9)
    n, d = 96, 32
    q, k, v = rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d)), rng.standard_normal((n, d))
    s = 0.2 * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    l = p.sum(axis=1, keepdims=True)
    pb = p.reshape(n, n // 32, 32)
    e = np.floor(np.log2(pb.max(-1, keepdims=True))) - 7  # block max lands in [128, 256)
    pq = e4m3_decode(e4m3_encode(pb * np.exp2(-e))) * np.exp2(e)
    o_q = (pq.reshape(n, n) / l) @ v
    o = (p / l) @ v
    bound = p_rounding_bound(q, k, v, 0.2)
    slack = 2.0 ** -13 * np.abs(v).max()  # values far below a block's max may be subnormal
    assert np.all(np.abs(o_q - o) <= bound + slack)
    assert np.abs(o_q - o).max() > 0.05 * bound.max()  # the rounding really happened


# --------------------------------------------------------------------------
# planted mistakes
# --------------------------------------------------------------------------

def _encode_truncating(x):  # rounds toward zero instead of to nearest
    mags = e4m3_decode(np.arange(0x7F))
    a = np.minimum(np.abs(np.asarray(x, dtype=np.float64)), 448.0)
    idx = np.searchsorted(mags, a, side="right") - 1
    return np.where(np.asarray(x) < 0, idx | 0x80, idx).astype(np.uint8)


def _scale_code_off_by_one(amax):  # one binade too small: the block max overflows E4M3
    return (np.asarray(mx_scale_code(amax)).astype(np.int64) - 1).astype(np.uint8)


def test_pins_catch_truncating_encoder():
    xs = np.array([1.1, 1.2, 300.0, 0.003])
    want = np.array([_brute_encode(float(x)) for x in xs], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(xs), want)
    assert not np.array_equal(_encode_truncating(xs), want)


def test_pins_catch_scale_off_by_one():
    got = _scale_code_off_by_one([1.0, 448.0, 449.0])
    assert not np.array_equal(got, np.array([119, 127, 128], dtype=np.uint8))
    assert np.array_equal(mx_scale_code([1.0, 448.0, 449.0]), np.array([119, 127, 128], dtype=np.uint8))
