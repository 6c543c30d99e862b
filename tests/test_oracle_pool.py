"""CPU checks of the GPU tests' oracle helpers (tests/oracle_pool.py).

backward_given_o is the oracle gradient with the row terms D_i = dO_i . O_i
taken from a given O (the backward's input) rather than the exact output. It
is built from oracle calls; these checks pin it: with the exact O it is the
exact gradient, dV never moves, and for one query the shift of dQ and dK has
the closed form of a single-row softmax written out here.
"""

import numpy as np

from oracle import attention_backward, attention_forward
from oracle_pool import backward_given_o


def _inputs(nq, nk, d, seed):
    rng = np.random.default_rng(seed)
    q, do = rng.standard_normal((nq, d)), rng.standard_normal((nq, d))
    k, v = rng.standard_normal((nk, d)), rng.standard_normal((nk, d))
    return q, k, v, do


def test_exact_o_gives_the_exact_gradient():
    for causal in (False, True):
        q, k, v, do = _inputs(9, 6, 8, seed=1)
        o, _ = attention_forward(q, k, v, 0.4, causal=causal)
        for a, b in zip(attention_backward(q, k, v, do, 0.4, causal=causal),
                        backward_given_o(q, k, v, o, do, 0.4, causal=causal)):
            assert np.array_equal(a, b)


def test_given_o_moves_dq_dk_not_dv():
    q, k, v, do = _inputs(5, 7, 8, seed=2)
    o, _ = attention_forward(q, k, v, 0.4)
    o2 = o + 1e-2 * np.random.default_rng(3).standard_normal(o.shape)
    exact = attention_backward(q, k, v, do, 0.4)
    given = backward_given_o(q, k, v, o2, do, 0.4)
    assert np.array_equal(exact[2], given[2])
    assert np.abs(exact[0] - given[0]).max() > 1e-6 and np.abs(exact[1] - given[1]).max() > 1e-6


def test_one_query_closed_form():
    # One query: p = softmax(scale k q), D = dO . O. Taking D from O + e
    # shifts dS_j = p_j (dP_j - D) by -p_j (dO . e), so dQ shifts by
    # -scale (dO . e) sum_j p_j k_j and dK_j by -scale (dO . e) p_j q.
    q, k, v, do = _inputs(1, 6, 8, seed=4)
    scale = 0.7
    o, _ = attention_forward(q, k, v, scale)
    e = 1e-2 * np.random.default_rng(5).standard_normal(o.shape)
    s = scale * (k @ q[0])
    p = np.exp(s - s.max())
    p /= p.sum()
    t = float(do[0] @ e[0])
    exact = attention_backward(q, k, v, do, scale)
    given = backward_given_o(q, k, v, o + e, do, scale)
    assert np.allclose(given[0] - exact[0], -scale * t * (p @ k)[None, :], rtol=1e-10, atol=1e-13)
    assert np.allclose(given[1] - exact[1], -scale * t * p[:, None] * q[0][None, :], rtol=1e-10, atol=1e-13)
