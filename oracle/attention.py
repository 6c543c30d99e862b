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
    pages only say it recomputes tile by tile from saved statistics);
  * causal attention (named by the Lecture 17 page at the end of §8.3 as
    something a real kernel must handle, without a definition) lets query i
    of N_q see key j of N_k iff j <= i + (N_k - N_q): the queries are the
    last N_q positions of the key sequence, which for N_q = N_k is the usual
    j <= i;
  * a query that sees no key at all (causal with N_q > N_k) has O = 0 and
    LSE = -inf: the log of an empty sum, and a part that adds nothing when
    partial results are merged;
  * partial results over disjoint key sets merge by the same rescaling as
    the online update (see merge_partials).
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


def causal_visible(n_q, n_k):
    """Boolean [n_q, n_k]: True where query i may attend key j, i.e. j <= i + n_k - n_q.

    The reading of "causal attention" (Lecture 17 page, end of §8.3) taken
    here: the N_q queries are the last N_q positions of the N_k keys.
    """
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i + (n_k - n_q)


def _masked_scores(qq, kk, scale, causal):
    s = scale * (qq @ kk.T)
    if causal:
        s = np.where(causal_visible(s.shape[0], s.shape[1]), s, -np.inf)
    return s


def _row_softmax(s):
    """(P, m, l) of each score row; a row of -inf only gives P = 0, m = -inf, l = 0."""
    m = s.max(axis=1, keepdims=True)
    m_shift = np.where(np.isfinite(m), m, 0.0)  # exp(-inf - 0) = 0 for an empty row
    e = np.exp(s - m_shift)
    l = e.sum(axis=1, keepdims=True)
    p = np.divide(e, l, out=np.zeros_like(e), where=l > 0)
    return p, m, l


def attention_forward(q, k, v, scale, causal=False):
    """O = softmax(scale * Q K^T) V and LSE, by the definition.

    [L17] §8.1 gives Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V; §8.3
    gives the softmax of a score row with the row maximum subtracted before
    exponentiating for stability. Steps, per (batch, head):
      S = scale * Q K^T (-inf where causal masks a key);  m_i = max_j S_ij;
      E = exp(S - m);  l_i = sum_j E_ij;  P = E / l;  O = P V;
      LSE_i = m_i + ln l_i.
    q is [..., N_q, d], k [..., N_k, d], v [..., N_k, d_v]. A row with no
    visible key gives O = 0, LSE = -inf. Returns (O [..., N_q, d_v],
    LSE [..., N_q]) in float64.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    o = np.empty(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    lse = np.empty(q.shape[:-1], dtype=np.float64)
    for idx in _slices(q.shape):
        s = _masked_scores(q[idx], k[idx], scale, causal)
        p, m, l = _row_softmax(s)
        o[idx] = p @ v[idx]
        with np.errstate(divide="ignore"):
            lse[idx] = (m + np.log(l))[:, 0]
    return o, lse


def attention_backward(q, k, v, do, scale, causal=False):
    """Exact gradients (dQ, dK, dV) of L = sum(O * dO) for O = attention(Q,K,V).

    The pages ([N5] §7.2 item 3; [R5] "FlashAttention 解析" ②) say only that
    the backward pass keeps no N x N matrix and recomputes it from saved
    statistics; they print no backward equations. The plainest reading is
    the exact gradient of the forward definition, written out by the chain
    rule through O = P V and the row softmax P = softmax(scale * Q K^T):
      dV = P^T dO;   dP = dO V^T;   D_i = sum_j P_ij dP_ij;
      dS = P * (dP - D);   dQ = scale * dS K;   dK = scale * dS^T Q.
    A masked key has P_ij = 0 and so dS_ij = 0; a row with no visible key
    contributes nothing. Returns float64 arrays shaped like q, k, v.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for idx in _slices(q.shape):
        s = _masked_scores(q[idx], k[idx], scale, causal)
        p, _, _ = _row_softmax(s)
        dv[idx] = p.T @ do[idx]
        dp = do[idx] @ v[idx].T
        d_row = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - d_row)
        dq[idx] = scale * (ds @ k[idx])
        dk[idx] = scale * (ds.T @ q[idx])
    return dq, dk, dv


def online_softmax_forward(q, k, v, scale, tile, causal=False):
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
    of attention_forward, used to pin it. With causal masking a row that has
    seen no visible key yet keeps (m, l, o) = (-inf, 0, 0) (the update is
    skipped for it: alpha = 1, p = 0), and a row that never sees one ends
    with O = 0, LSE = -inf.
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
        vis = causal_visible(n_q, n_k) if causal else None
        for j0 in range(0, n_k, tile):
            s = scale * (qq @ kk[j0:j0 + tile].T)
            if causal:
                s = np.where(vis[:, j0:j0 + tile], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1, keepdims=True))
            seen = np.isfinite(m_new)  # rows with at least one visible key so far
            m_ref = np.where(seen, m_new, 0.0)
            alpha = np.where(seen, np.exp(m - m_ref), 1.0)
            p = np.exp(s - m_ref)  # exactly 0 for masked keys
            l = alpha * l + p.sum(axis=1, keepdims=True)
            o = alpha * o + p @ vv[j0:j0 + tile]
            m = m_new
        o_out[idx] = np.divide(o, l, out=np.zeros_like(o), where=l > 0)
        with np.errstate(divide="ignore"):
            lse[idx] = (m + np.log(l))[:, 0]
    return o_out, lse


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key sets into the result over their union.

    The CS336 Lecture 5 transcript ([R5], FlashAttention passage) describes
    computing the softmax of one tile, writing the partial result back to
    global memory and continuing; [L17] §8.3's update rescales a running
    state by e^(m - m'). For a part r holding O_r = o_r / l_r and
    LSE_r = m_r + ln l_r (o_r = sum of e^(s - m_r) v over its keys), the
    union has l = sum_r e^(m_r) l_r, i.e.
      LSE = ln sum_r e^(LSE_r),   O = sum_r e^(LSE_r - LSE) O_r,
    taken here with the largest LSE_r subtracted first. Parts with
    LSE_r = -inf (no visible key) weigh 0; if every part is empty the result
    is O = 0, LSE = -inf.
    o_parts: [P, ..., N, d]; lse_parts: [P, ..., N]. Returns (O, LSE) float64.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    if o_parts.shape[:-1] != lse_parts.shape or o_parts.shape[0] < 1:
        raise ValueError("expected o_parts [P, ..., N, d] and lse_parts [P, ..., N] with P >= 1")
    mx = lse_parts.max(axis=0)
    shift = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lse_parts - shift)  # 0 for empty parts
    total = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = shift + np.log(total)
    lse = np.where(total > 0, lse, -np.inf)
    wn = np.divide(w, total, out=np.zeros_like(w), where=total > 0)
    o = (wn[..., None] * o_parts).sum(axis=0)
    return o, lse


# ---------------------------------------------------------------------------
# Brute force on tiny inputs: pure Python loops and math.exp, no NumPy
# arithmetic, so that a mistake in the vectorised oracle cannot hide in a
# shared library call.
# ---------------------------------------------------------------------------

def _tolist2(x):
    return [[float(t) for t in row] for row in np.asarray(x, dtype=np.float64)]


def brute_force_forward(q, k, v, scale, causal=False):
    """Single-head attention by explicit loops ([L17] §8.1 definition).

    q: [Nq, d], k: [Nk, d], v: [Nk, dv] (array-likes). Returns Python lists
    (O as Nq lists of dv floats, LSE as Nq floats). The softmax uses the
    max-shifted form of [L17] §8.3 so that it cannot overflow. With causal,
    query i only loops over keys j <= i + Nk - Nq; with none, O_i = 0 and
    LSE_i = -inf.
    """
    Q, K, V = _tolist2(q), _tolist2(k), _tolist2(v)
    n_q, n_k, dv = len(Q), len(K), len(V[0])
    out, lse = [], []
    for i, qi in enumerate(Q):
        keys = [j for j in range(n_k) if not causal or j <= i + n_k - n_q]
        if not keys:
            out.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        s = {j: scale * sum(a * b for a, b in zip(qi, K[j])) for j in keys}
        m = max(s.values())
        e = {j: math.exp(s[j] - m) for j in keys}
        den = sum(e.values())
        out.append([sum(e[j] * V[j][c] for j in keys) / den for c in range(dv)])
        lse.append(m + math.log(den))
    return out, lse


def brute_force_backward(q, k, v, do, scale, h=1e-6, causal=False):
    """Gradients of L = sum(O * dO) by central finite differences.

    This deliberately does not use the chain-rule formulas of
    attention_backward: each input element is perturbed by +-h and the
    brute-force forward is re-evaluated, so it is an independent check of
    those formulas (truncation error O(h^2), rounding error O(eps/h)).
    Returns (dQ, dK, dV) as nested Python lists.
    """
    Q, K, V, dO = _tolist2(q), _tolist2(k), _tolist2(v), _tolist2(do)

    def loss(Qx, Kx, Vx):
        o, _ = brute_force_forward(Qx, Kx, Vx, scale, causal)
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
