"""Float64 CPU oracle for MXFP8 attention (test infrastructure only).

Source: the CS336 Lecture 5 transcript ([R5]) on low-precision formats: FP8
comes as E4M3 (4 exponent bits, 3 mantissa bits) or E5M2; a single FP32
scale per tensor copes badly with parts of a matrix of very different
magnitude, so MXFP8 gives every 32 consecutive elements their own scale, a
power of two stored in 8 bits, and uses E4M3 elements. The transcript also
poses the catch of the design: the 32-element blocks run along one dimension
of the matrix, so an operand used transposed (V in O = P V, reduced over
keys) needs a copy quantized along the other dimension.

Readings taken here (the pages give no bit-level definition):
  * E4M3 is the 8-bit format with sign, 4 exponent bits (bias 7) and 3
    mantissa bits, exponent field 0 for subnormals (m * 2^-9), no infinity,
    and S.1111.111 as NaN, so the largest finite value is 448;
  * an element is rounded to the nearest E4M3 value, ties to even mantissa,
    and magnitudes beyond 448 saturate to 448;
  * a block's scale is the smallest power of two 2^e with amax <= 448 * 2^e,
    amax its largest magnitude (so amax / scale lies in (224, 448]: the
    block's largest element uses the top binade of E4M3 and nothing
    saturates), stored as the biased exponent byte e + 127, clamped to
    0..254; an all-zero block gets byte 0. With amax = m 2^x, m in [1, 2),
    e = x - 8 if m <= 1.75 and x - 7 otherwise;
  * MXFP8 attention is attention (attention.py) evaluated on the dequantized
    inputs q_hat, k_hat, v_hat; the kernel's further approximation (P
    rounded to E4M3 in 32-key blocks before O = P V) is not part of this
    definition and is bounded by p_rounding_bound().
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_decode(codes):
    """Values of E4M3 codes (uint8 array-like); NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * np.exp2(e.astype(np.float64) - 10.0))
    v = np.where((e == 15) & ((c & 7) == 7), np.nan, v)
    return s * v


def _all_values():
    codes = np.arange(128)
    vals = e4m3_decode(codes)
    keep = ~np.isnan(vals)
    return codes[keep], vals[keep]  # non-negative codes 0x00 .. 0x7e, increasing values


_POS_CODES, _POS_VALS = _all_values()


def e4m3_encode(x):
    """Round float64 values to E4M3 codes: nearest, ties to even mantissa, saturating at 448."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no MXFP8 encoding here")
    a = np.minimum(np.abs(x), E4M3_MAX)
    # index of the largest representable value <= a, and the next one up
    hi = np.searchsorted(_POS_VALS, a, side="left")
    hi = np.minimum(hi, len(_POS_VALS) - 1)
    lo = np.where(_POS_VALS[hi] > a, hi - 1, hi)
    up = np.minimum(lo + 1, len(_POS_VALS) - 1)
    vlo, vup = _POS_VALS[lo], _POS_VALS[up]
    dlo, dup = a - vlo, vup - a
    even_lo = (_POS_CODES[lo] & 1) == 0
    pick_up = (dup < dlo) | ((dup == dlo) & ~even_lo & (up != lo))
    code = np.where(pick_up, _POS_CODES[up], _POS_CODES[lo]).astype(np.int64)
    neg = (x < 0) | ((x == 0) & np.signbit(x))
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def mx_scale_code(amax):
    """E8M0 scale byte of a block with largest magnitude amax (0 for amax = 0).

    The smallest e with amax <= 448 * 2^e, biased by 127 and clamped to 0..254.
    frexp gives amax = f * 2^x exactly with f in [0.5, 1): floor(log2 amax) =
    x - 1 and the significand is 2f, so e = x - 9 + (2f > 1.75).
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, x = np.frexp(np.where(amax > 0, amax, 1.0))
    e = (x.astype(np.int64) - 9) + (2.0 * f > 1.75)
    code = np.clip(e + 127, 0, 254)
    return np.where(amax > 0, code, 0).astype(np.uint8)


def mx_quantize(x, axis=-1):
    """MXFP8 (E4M3 elements, one E8M0 scale per 32 consecutive elements along `axis`).

    The length along `axis` must be a multiple of 32. Returns (codes uint8,
    shape of x; scales uint8, shape of x with that axis divided by 32).
    """
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError("the blocked axis must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))
    sc = mx_scale_code(np.abs(xb).max(axis=-1))
    mult = np.exp2(127.0 - sc.astype(np.float64))  # 1 / scale
    codes = e4m3_encode(xb * mult[..., None]).reshape(x.shape)
    return np.moveaxis(codes, -1, axis), np.moveaxis(sc, -1, axis)


def mx_dequantize(codes, scales, axis=-1):
    """Exact float64 values of MXFP8 data (inverse of the layout of mx_quantize)."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1)
    n = c.shape[-1]
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (n // BLOCK, BLOCK))
    vals = vals * np.exp2(s.astype(np.float64) - 127.0)[..., None]
    return np.moveaxis(vals.reshape(c.shape), -1, axis)


def attention_forward_mxfp8(q8, q_sc, k8, k_sc, vt8, vt_sc, scale):
    """MXFP8 attention: O, LSE of attention on the dequantized inputs.

    q8, k8: [..., N, d] codes with scales [..., N, d/32] (blocks along d);
    vt8: [..., d, N] codes of V transposed with scales [..., d, N/32]
    (blocks along the keys). Returns float64 (O [..., N, d], LSE [..., N]).
    """
    q = mx_dequantize(q8, q_sc)
    k = mx_dequantize(k8, k_sc)
    v = np.swapaxes(mx_dequantize(vt8, vt_sc), -1, -2)
    return attention_forward(q, k, v, scale)


def p_rounding_bound(q, k, v, scale):
    """Per-element bound on |O_kernel - O| from rounding P to E4M3 before O = P V.

    Each normal E4M3 value carries 3 mantissa bits, so rounding to nearest
    changes a probability by at most 2^-4 of itself; with O_ic = sum_j P_ij
    v_jc and every P_ij perturbed by at most 2^-4 P_ij, |delta O_ic| <=
    2^-4 sum_j P_ij |v_jc|. Returns that bound ([..., N, d], float64).
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    s = scale * (q @ np.swapaxes(k, -1, -2))
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return 2.0 ** -4 * (p @ np.abs(v))
