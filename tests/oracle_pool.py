"""Whole-output oracle evaluation for the GPU parity tests at full workload sizes.

The float64 oracle works on one (batch, head) slice at a time and is exact
row by row for the unmasked forward (row i of O and LSE depends only on
query i), so a full-size comparison splits the work into independent tasks
(a head, or a block of query rows of a head) and runs them in a thread pool:
NumPy's matrix products and element-wise passes release the interpreter
lock, and each worker runs its products on one BLAS thread so the pool does
not oversubscribe the host. Nothing here computes attention itself; every
number comes from oracle/.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from threadpoolctl import threadpool_limits

from oracle import attention_backward, attention_forward


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _run(tasks):
    """Results of the zero-argument callables in `tasks`, in order."""
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            return list(ex.map(lambda f: f(), tasks))


def forward_all(q, k, v, scale, causal=False, row_block=None):
    """Oracle O [B, H, Nq, d] and LSE [B, H, Nq] for float64 q, k, v [B, H, N, d].

    row_block splits each head's queries into blocks of that many rows (the
    unmasked forward only: with the causal mask a row's visible keys depend on
    its index within the whole query sequence).
    """
    B, H, Nq, _ = q.shape
    if row_block is not None and causal:
        raise ValueError("row blocks are only exact for the unmasked forward")
    rb = Nq if row_block is None else row_block
    spans = [(b, h, r, min(Nq, r + rb)) for b in range(B) for h in range(H) for r in range(0, Nq, rb)]
    out = _run([lambda s=s: attention_forward(q[s[0], s[1], s[2]:s[3]], k[s[0], s[1]], v[s[0], s[1]],
                                              scale, causal=causal) for s in spans])
    o = np.empty(q.shape[:3] + (v.shape[3],))
    lse = np.empty(q.shape[:3])
    for (b, h, r0, r1), (ro, rl) in zip(spans, out):
        o[b, h, r0:r1] = ro
        lse[b, h, r0:r1] = rl
    return o, lse


def backward_given_o(q, k, v, o, do, scale, causal=False):
    """Oracle dQ, dK, dV of one head when the row terms D_i = dO_i . O_i are
    taken from the given O, the output the backward is handed (the forward's
    stored, rounded result), instead of the exact one.

    The pages print no backward; the reading here (as in the kernel) takes D
    from the O passed in. dS = P * (dP - D) is linear in D, so with
    delta_i = dO_i . (O_i - O_exact_i) the exact gradients move by
    dQ: -scale * delta_i * (P K)_i and dK: -scale * P^T (delta * Q), dV not at
    all. Both terms are oracle evaluations: P K is the attention output with K
    in place of V, and P^T Y is dV for the output gradient Y. When the given O
    is the exact one, delta = 0 and this is attention_backward itself.
    """
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal=causal)
    o_exact, _ = attention_forward(q, k, v, scale, causal=causal)
    delta = np.sum(do * (o - o_exact), axis=-1, keepdims=True)
    pk, _ = attention_forward(q, k, k, scale, causal=causal)
    _, _, pty = attention_backward(q, k, v, delta * q, scale, causal=causal)
    return dq - scale * delta * pk, dk - scale * pty, dv


def backward_all(q, k, v, o, do, scale, causal=False):
    """backward_given_o for every head of float64 [B, H, N, d] inputs."""
    B, H = q.shape[:2]
    heads = [(b, h) for b in range(B) for h in range(H)]
    out = _run([lambda bh=bh: backward_given_o(q[bh], k[bh], v[bh], o[bh], do[bh], scale, causal=causal)
                for bh in heads])
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for bh, (gq, gk, gv) in zip(heads, out):
        dq[bh], dk[bh], dv[bh] = gq, gk, gv
    return dq, dk, dv
