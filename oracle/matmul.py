"""Float64 CPU oracle for the matrix product C = A B^T (test infrastructure only).

The Lecture 17 page §2.1 defines the matrix product element by element,
C_ij = sum_k A_ik B_kj, and §5.3 counts it as 2MKN floating-point operations.
Here the second operand is given transposed (B is [N, K], so that both
operands are contiguous along the reduction index, as Q and K are in
S = Q K^T): C_ij = sum_k A_ik B_jk. NumPy's float64 matmul serves as the
step (a library primitive); brute_force_matmul_nt is the same sum in pure
Python loops, used to pin it.
"""

from __future__ import annotations

import numpy as np


def matmul_nt(a, b):
    """C = A B^T in float64 for A [M, K] and B [N, K]."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("expected A [M, K] and B [N, K]")
    return a @ b.T


def brute_force_matmul_nt(a, b):
    """C_ij = sum_k A_ik B_jk by explicit loops (Lecture 17 page §2.1)."""
    A = [[float(x) for x in row] for row in np.asarray(a, dtype=np.float64)]
    B = [[float(x) for x in row] for row in np.asarray(b, dtype=np.float64)]
    return [[sum(A[i][k] * B[j][k] for k in range(len(A[i]))) for j in range(len(B))]
            for i in range(len(A))]
