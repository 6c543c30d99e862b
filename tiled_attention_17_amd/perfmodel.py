"""Work, traffic and roofline arithmetic for the attention kernels.

Counting rules, from the Lecture 17 page (§5.3: a matmul of M x K by K x N
costs about 2MKN floating-point operations and, with 16-bit elements read
once and written once, at least 2(MK + KN + MN) bytes; §6.1: arithmetic
intensity is FLOPs per byte moved at a stated memory level; §6.2: the
roofline bound is min(peak, bandwidth x intensity)) and from the CS336
Lecture 5 notes §6.2 (wave quantization: tiles beyond a whole number of
waves over the compute units leave the chip mostly idle).
"""

from __future__ import annotations

import math

# MI355X (gfx950) published figures.
MI355X_CUS = 256
MI355X_XCDS = 8
MI355X_CLOCK_HZ = 2.4e9
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_PEAK_FLOPS = {
    "bf16": 2.5e15,   # dense MFMA
    "fp16": 2.5e15,
    "fp32": 157.3e12,  # fp32 matrix
    "fp8": 5.0e15,     # dense MFMA (E4M3 / MXFP8)
}


def matmul_flops(m, k, n):
    return 2 * m * k * n


def matmul_min_bytes(m, k, n, elem_bytes=2):
    return elem_bytes * (m * k + k * n + m * n)


def intensity(flops, nbytes):
    return flops / nbytes


def roofline_bound(peak_flops, bandwidth, ai):
    return min(peak_flops, bandwidth * ai)


def tiles(m, n, tile_m, tile_n):
    return math.ceil(m / tile_m) * math.ceil(n / tile_n)


def waves(n_tiles, units):
    return math.ceil(n_tiles / units)


def tail_tiles(n_tiles, units):
    """Tiles in the last, partial wave (0 when the tiles fill whole waves)."""
    r = n_tiles % units
    return r


def attn_fwd_flops(B, H, N, d, Nk=None):
    """Two matmuls per head: S = Q K^T and O = P V, 2*N*Nk*d each."""
    Nk = N if Nk is None else Nk
    return 4 * B * H * N * Nk * d


def attn_bwd_flops(B, H, N, d, Nk=None):
    """Five matmuls per head: recomputed Q K^T, P^T dO, dO V^T, dS K, dS^T Q."""
    Nk = N if Nk is None else Nk
    return 10 * B * H * N * Nk * d


def attn_fwd_bytes(B, H, N, d, elem_bytes):
    """Read Q, K, V once, write O once, write the fp32 LSE once."""
    return B * H * (4 * N * d * elem_bytes + 4 * N)


def attn_bwd_bytes(B, H, N, d, elem_bytes):
    """Read Q, K, V, O, dO and write dQ, dK, dV once; LSE read, row term D written and read (fp32)."""
    return B * H * (8 * N * d * elem_bytes + 3 * N * 4)


def visible_pairs(Nq, Nk, causal):
    """(query, key) pairs the attention covers: all Nq * Nk, or under the causal
    mask (query i sees key j iff j <= i + Nk - Nq) sum_i clamp(i + Nk - Nq + 1, 0, Nk)."""
    if not causal:
        return Nq * Nk
    off = Nk - Nq
    # rows i < -off see nothing; rows from Nq - 1 - ... see all Nk keys once i + off + 1 >= Nk
    lo = max(0, -off)                  # first row with a visible key
    full = max(lo, min(Nq, Nk - off - 1))  # first row that sees every key
    ramp = sum(range(lo + off + 1, full + off + 1)) if full > lo else 0
    return ramp + (Nq - full) * Nk


def attn_fwd_flops_masked(B, H, Nq, Nk, d, causal):
    """Two matmuls over the visible (query, key) pairs: 4 d FLOPs per pair."""
    return 4 * B * H * d * visible_pairs(Nq, Nk, causal)


def attn_bwd_flops_masked(B, H, Nq, Nk, d, causal):
    """Five matmuls over the visible pairs: 10 d FLOPs per pair."""
    return 10 * B * H * d * visible_pairs(Nq, Nk, causal)


def attn_fwd_bytes_ex(B, H, Nq, Nk, d, elem_bytes):
    """Read Q and K, V once, write O once, write the fp32 LSE once."""
    return B * H * (2 * Nq * d * elem_bytes + 2 * Nk * d * elem_bytes + 4 * Nq)
