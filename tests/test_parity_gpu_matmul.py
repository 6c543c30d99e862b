"""GPU parity of the matrix product C = A B^T (attn_matmul_nt) against the float64 oracle.

Bar (derived from the arithmetic): products of two bf16 values are exact in
fp32; the kernel sums the K of them in fp32 (unit roundoff 2^-24), which
errs by at most K 2^-24 sum_k |a_k b_k| in any order of summation, and then
rounds C once to bf16 (round to nearest even, unit roundoff u = 2^-8). So
every element must satisfy
  |C - C_ref| <= 2^-8 |C_ref| + (1 + 2^-8) 1.01 K 2^-24 (|A| |B|^T),
the 1.01 covering the second-order term of the summation bound for K up to
4096. Integer-valued inputs whose sums are exact in bf16 must come back
bit-exact.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import tiled_attention_17_amd as ta  # noqa: E402
from oracle import matmul_nt  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ta.library()


def _operands(m, n, k, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn((m, k), generator=g).to(torch.bfloat16)
    b = torch.randn((n, k), generator=g).to(torch.bfloat16)
    return a, b


def _check(a, b, c, rows=None):
    a64, b64 = a.double().numpy(), b.double().numpy()
    if rows is not None:
        a64 = a64[rows]
    ref = matmul_nt(a64, b64)
    absdot = matmul_nt(np.abs(a64), np.abs(b64))
    got = c.double().cpu().numpy()
    if rows is not None:
        got = got[rows]
    assert np.all(np.isfinite(got))
    k = a64.shape[1]
    bound = 2.0 ** -8 * np.abs(ref) + (1 + 2.0 ** -8) * 1.01 * k * 2.0 ** -24 * absdot
    bad = np.abs(got - ref) > bound
    assert not bad.any(), f"{bad.sum()} elements outside the bar; max err {np.abs(got - ref).max():.3e}"


@pytest.mark.parametrize("m,n,k", [(1, 1, 8), (128, 128, 64), (200, 300, 72), (513, 1000, 520),
                                   (1000, 513, 64), (256, 256, 8), (129, 127, 136), (64, 4096, 256)])
def test_matmul_small_and_ragged(m, n, k):
    a, b = _operands(m, n, k, m + n + k)
    c = ta.attn_matmul_nt(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    _check(a, b, c)


def test_matmul_integer_inputs_bit_exact():
    g = torch.Generator().manual_seed(3)
    a = torch.randint(-2, 3, (300, 64), generator=g).to(torch.bfloat16)
    b = torch.randint(-2, 3, (257, 64), generator=g).to(torch.bfloat16)
    c = ta.attn_matmul_nt(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    ref = a.double() @ b.double().T  # |C| <= 256: exact in bf16
    assert torch.equal(c.double().cpu(), ref)


def test_matmul_k_zero_and_empty():
    a = torch.empty((70, 0), dtype=torch.bfloat16, device="cuda")
    b = torch.empty((90, 0), dtype=torch.bfloat16, device="cuda")
    c = ta.attn_matmul_nt(a, b)
    e = ta.attn_matmul_nt(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                          torch.ones((5, 64), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert c.shape == (70, 90) and torch.all(c == 0) and e.shape == (0, 5)


@pytest.mark.parametrize("size", [4096, 4097])
def test_matmul_sweep_sizes_sampled(size):
    # the sweep's sizes on each side of a whole number of tile rounds
    a, b = _operands(size, size, 1024, size)
    c = ta.attn_matmul_nt(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(size)
    rows = np.unique(np.concatenate([[0, 127, 128, size - 1], rng.integers(0, size, 60)]))
    _check(a, b, c, rows=rows)
