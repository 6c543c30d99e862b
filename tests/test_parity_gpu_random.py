"""GPU parity on a seeded random sweep of forward and backward configurations.

Each case draws batch, heads, query and key counts (from 1 to past a thousand,
so tile edges and ragged tails fall anywhere), d, dtype, the causal mask, the
number of key splits (0 = the library's choice) and the spread of Q, runs
attn_fwd_ex (and, for bf16, attn_bwd_ex) through the C ABI, and compares every
head with the float64 CPU oracle. The cases are drawn once from a fixed seed,
so the sweep is the same on every run.

Bars. bf16 O: max abs error <= 2e-2 (and <= 2e-2 max|ref| + 1e-4), as in the
other parity tests: |O| stays below ~4 here, so the bf16 rounding of O itself
(unit roundoff u = 2^-8, 8 significant bits) is at most ~0.016. bf16 dQ, dK,
dV: <= 2e-2 + 2u max|ref| = 2e-2 + 2^-7 max|ref|: one u for the rounding of
the result, one for the bf16 rounding of the P and dS operands (errors of
independent sign over the summed terms, which add up to about u |result|).
With Q ~ N(0, 3^2) the gradients reach |dK| ~ 16, where the rounding of the
result alone is up to u 16 = 0.06, more than 2e-2. The relative check
2e-2 max|ref| + 1e-4 keeps a wrongly scaled result from passing (the 1e-4
floor is for results that vanish analytically, such as dK with a single key,
which come back at rounding level). fp32 O: <= 1e-5. LSE <= 1e-3 absolute.
Rows that see no key come back as exactly O = 0, LSE = -inf, dQ = 0.

Gradient reference: the oracle gradient with the row terms D_i = dO_i . O_i
taken from the O the backward is handed (oracle_pool.backward_given_o), as
the kernel takes them. The exact gradient differs from it by a term from the
bf16 rounding of O, which exceeds the relative check where cancellation
leaves a gradient small (one query against a peaked softmax: |dQ| ~ 7e-3 with
a 2.5e-3 shift).
"""

import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import tiled_attention_17_amd as ta  # noqa: E402
from oracle import attention_forward  # noqa: E402
from oracle_pool import backward_given_o  # noqa: E402
from tiled_attention_17_amd.workloads import Workload, make_inputs, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
BF16_REL = 2e-2
FP32_TOL = 1e-5
LSE_TOL = 1e-3


def _draw_cases(n, seed):
    rng = random.Random(seed)

    def length():
        return rng.choice([1, rng.randint(2, 64), rng.randint(65, 400), rng.randint(401, 1100)])

    cases = []
    for i in range(n):
        dtype = "bf16" if rng.random() < 0.8 else "fp32"
        case = dict(B=rng.choice([1, 2]), H=rng.choice([1, 2, 3]), Nq=length(), Nk=length(),
                    d=rng.choice([64, 128]), dtype=dtype, causal=rng.random() < 0.5,
                    splits=rng.choice([1, 1, 2, 3, 0]), q_std=rng.choice([1.0, 1.0, 3.0]),
                    bwd=dtype == "bf16" and rng.random() < 0.6, seed=1000 + i)
        cases.append(case)
    return cases


CASES = _draw_cases(96, seed=20261203)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ta.library()


BF16_U = 2.0 ** -8  # unit roundoff of bf16 round-to-nearest-even (8 significant bits)
GRAD_ROUNDING = 2 * BF16_U  # result rounding plus the P and dS operand roundings


def _assert_close(name, got, want, tol, rel, grad=False):
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    if not want.size:
        return
    err = float(np.max(np.abs(got - want)))
    scale = float(np.max(np.abs(want)))
    bound = tol + (GRAD_ROUNDING * scale if grad else 0.0)
    assert err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e} (max|ref| {scale:.3e})"
    if rel is not None:
        assert err <= rel * scale + 1e-4, f"{name}: max err {err:.3e} > {rel} * max|ref| {scale:.3e} + 1e-4"


def _case_id(c):
    return (f"B{c['B']}H{c['H']}_q{c['Nq']}_k{c['Nk']}_d{c['d']}_{c['dtype']}"
            f"{'_causal' if c['causal'] else ''}_s{c['splits']}_std{c['q_std']:g}{'_bwd' if c['bwd'] else ''}")


@pytest.mark.parametrize("case", CASES, ids=[_case_id(c) for c in CASES])
def test_random_configuration(case):
    c = case
    w = Workload(_case_id(c), c["B"], c["H"], c["Nq"], c["d"], c["dtype"], seed=c["seed"], q_std=c["q_std"],
                 n_k=c["Nk"], causal=c["causal"])
    x = {k: t.cuda() for k, t in make_inputs(w, with_grad_output=c["bwd"]).items()}
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=c["causal"], num_splits=c["splits"])
    if c["bwd"]:
        dq, dk, dv = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=c["causal"])
    torch.cuda.synchronize()

    tol, rel = (BF16_TOL, BF16_REL) if c["dtype"] == "bf16" else (FP32_TOL, None)
    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    go, gl = to_f64(o), to_f64(lse)
    if c["bwd"]:
        do = to_f64(x["do"])
        grads = [to_f64(t) for t in (dq, dk, dv)]
    for (b, h) in np.ndindex(c["B"], c["H"]):
        ro, rl = attention_forward(q[b, h], k[b, h], v[b, h], w.scale, causal=c["causal"])
        empty = np.isneginf(rl)
        assert np.array_equal(np.isneginf(gl[b, h]), empty), f"LSE[{b},{h}]: rows without keys differ"
        assert np.all(go[b, h][empty] == 0), f"O[{b},{h}]: rows without keys are not 0"
        _assert_close(f"O[{b},{h}]", go[b, h], ro, tol, rel)
        if (~empty).any():
            err = float(np.max(np.abs(gl[b, h][~empty] - rl[~empty])))
            assert err <= LSE_TOL, f"LSE[{b},{h}]: max abs err {err:.3e} > {LSE_TOL:.1e}"
        if c["bwd"]:
            ref = backward_given_o(q[b, h], k[b, h], v[b, h], go[b, h], do[b, h], w.scale, causal=c["causal"])
            for name, got, want in zip(("dQ", "dK", "dV"), grads, ref):
                _assert_close(f"{name}[{b},{h}]", got[b, h], want, BF16_TOL, BF16_REL, grad=True)
            assert np.all(grads[0][b, h][empty] == 0), f"dQ[{b},{h}]: rows without keys are not 0"
