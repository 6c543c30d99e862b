"""Float64 CPU oracle for softmax attention (test infrastructure only).

Everything here works on NumPy float64 arrays laid out [..., N, d] (any
leading batch/head dimensions) and processes one (batch, head) slice at a
time, materialising the full N x N score and probability matrices -- the
very thing the fused GPU kernel avoids -- because that is the plain
definition.

Readings of the pages taken here (each also listed in the design notes):
  * scores are scale * q_i . k_j with the caller's scale (1/sqrt(d) in every
    workload), applied before the max shift and the exponential;
  * LSE_i = ln sum_j exp(scale * q_i . k_j), natural log;
  * the backward pass is the exact gradient of the forward definition (the
    pages only say it recomputes tile by tile from saved statistics).
"""

from __future__ import annotations

import math

import numpy as np


def _as_f64(x):
    a = np.asarray(x, dtype=np.float64)
    if a.ndim < 2:
        raise ValueError("expected an array of shape [..., N, d]")
    return a


def _slices(shape):
    """Index tuples over all leading (batch, head) dimensions."""
    return list(np.ndindex(*shape[:-2])) if len(shape) > 2 else [()]


def attention_forward(q, k, v, scale):
    """O = softmax(scale * Q K^T) V and LSE, by the definition.

    [L17] §8.1 gives Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V; §8.3
    gives the softmax of a score row with the row maximum subtracted before
    exponentiating for stability. Steps, per (batch, head):
      S = scale * Q K^T;  m_i = max_j S_ij;  E = exp(S - m);  l_i = sum_j E_ij;
      P = E / l;  O = P V;  LSE_i = m_i + ln l_i.
    Returns (O [..., N, d], LSE [..., N]) in float64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for idx in _slices(q.shape):
        s = scale * (q[idx] @ k[idx].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        p = e / l
        o[idx] = p @ v[idx]
        lse[idx] = (m + np.log(l))[:, 0]
    return o, lse


def attention_backward(q, k, v, do, scale):
    """Exact gradients (dQ, dK, dV) of L = sum(O * dO) for O = attention(Q,K,V).

    The pages ([N5] §7.2 item 3; [R5] "FlashAttention 解析" ②) say only that
    the backward pass keeps no N x N matrix and recomputes it from saved
    statistics; they print no backward equations. The plainest reading is
    the exact gradient of the forward definition, written out by the chain
    rule through O = P V and the row softmax P = softmax(scale * Q K^T):
      dV = P^T dO;   dP = dO V^T;   D_i = sum_j P_ij dP_ij;
      dS = P * (dP - D);   dQ = scale * dS K;   dK = scale * dS^T Q.
    Returns float64 arrays shaped like q, k, v.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for idx in _slices(q.shape):
        s = scale * (q[idx] @ k[idx].T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        dv[idx] = p.T @ do[idx]
        dp = do[idx] @ v[idx].T
        d_row = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - d_row)
        dq[idx] = scale * (ds @ k[idx])
        dk[idx] = scale * (ds.T @ q[idx])
    return dq, dk, dv


def online_softmax_forward(q, k, v, scale, tile):
    """Attention by the online softmax state update, over key tiles of width `tile`.

    [L17] §8.3: per query row keep (m, l, o) -- the running maximum score, the
    running sum of shifted exponentials and the running exponential-weighted
    sum of value rows -- starting from m = -inf, l = 0, o = 0. For each new
    tile of scores s:
      m' = max(m, max(s));  alpha = e^(m - m');  p = e^(s - m');
      l' = alpha * l + sum_j p_j;  o' = alpha * o + p V_tile;
    and after the last tile O = o / l. [R5] states the same correction of the
    running sum by exp(m_old - m_new). LSE = m + ln l (the statistic the
    backward pass reuses). This is an independent second path to the result
    of attention_forward, used to pin it.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if tile < 1:
        raise ValueError("tile width must be >= 1")
    n_k = k.shape[-2]
    o_out = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for idx in _slices(q.shape):
        qq, kk, vv = q[idx], k[idx], v[idx]
        n_q = qq.shape[0]
        m = np.full((n_q, 1), -np.inf)
        l = np.zeros((n_q, 1))
        o = np.zeros((n_q, vv.shape[1]))
        for j0 in range(0, n_k, tile):
            s = scale * (qq @ kk[j0:j0 + tile].T)
            m_new = np.maximum(m, s.max(axis=1, keepdims=True))
            alpha = np.exp(m - m_new)
            p = np.exp(s - m_new)
            l = alpha * l + p.sum(axis=1, keepdims=True)
            o = alpha * o + p @ vv[j0:j0 + tile]
            m = m_new
        o_out[idx] = o / l
        lse[idx] = (m + np.log(l))[:, 0]
    return o_out, lse


# ---------------------------------------------------------------------------
# Brute force on tiny inputs: pure Python loops and math.exp, no NumPy
# arithmetic, so that a mistake in the vectorised oracle cannot hide in a
# shared library call.
# ---------------------------------------------------------------------------

def _tolist2(x):
    return [[float(t) for t in row] for row in np.asarray(x, dtype=np.float64)]


def brute_force_forward(q, k, v, scale):
    """Single-head attention by explicit loops ([L17] §8.1 definition).

    q: [Nq, d], k: [Nk, d], v: [Nk, dv] (array-likes). Returns Python lists
    (O as Nq lists of dv floats, LSE as Nq floats). The softmax uses the
    max-shifted form of [L17] §8.3 so that it cannot overflow.
    """
    Q, K, V = _tolist2(q), _tolist2(k), _tolist2(v)
    out, lse = [], []
    for qi in Q:
        s = [scale * sum(a * b for a, b in zip(qi, kj)) for kj in K]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = sum(e)
        out.append([sum(e[j] * V[j][c] for j in range(len(K))) / den
                    for c in range(len(V[0]))])
        lse.append(m + math.log(den))
    return out, lse


def brute_force_backward(q, k, v, do, scale, h=1e-6):
    """Gradients of L = sum(O * dO) by central finite differences.

    This deliberately does not use the chain-rule formulas of
    attention_backward: each input element is perturbed by +-h and the
    brute-force forward is re-evaluated, so it is an independent check of
    those formulas (truncation error O(h^2), rounding error O(eps/h)).
    Returns (dQ, dK, dV) as nested Python lists.
    """
    Q, K, V, dO = _tolist2(q), _tolist2(k), _tolist2(v), _tolist2(do)

    def loss(Qx, Kx, Vx):
        o, _ = brute_force_forward(Qx, Kx, Vx, scale)
        return sum(o[i][c] * dO[i][c] for i in range(len(o)) for c in range(len(o[0])))

    def grad(which):
        mats = [Q, K, V]
        base = mats[which]
        g = [[0.0] * len(base[0]) for _ in base]
        for r in range(len(base)):
            for c in range(len(base[0])):
                plus = [[row[:] for row in mm] for mm in mats]
                minus = [[row[:] for row in mm] for mm in mats]
                plus[which][r][c] += h
                minus[which][r][c] -= h
                g[r][c] = (loss(*plus) - loss(*minus)) / (2.0 * h)
        return g

    return grad(0), grad(1), grad(2)
