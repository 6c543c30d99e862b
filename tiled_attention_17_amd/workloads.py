"""Seeded synthetic attention workloads (inputs only: no attention arithmetic).

This module is the one piece shared by the GPU path's tests/benchmark and the
CPU oracle's callers: it draws the input tensors. It computes nothing of the
method itself.

Recipe (the pages measure on no dataset, so these synthetic shapes are the
workload): a CPU torch.Generator seeded per workload draws Q, K, V and (for
the backward workload) dO, in that order, with torch.randn in float32; Q is
multiplied by its standard deviation (3 for the long-sequence workload, which
spreads the scores so the running max is rescaled often); the tensors are
then rounded to the workload dtype (round-to-nearest-even for bfloat16).
Layout is [B, H, N, d], contiguous, d innermost. The oracle consumes the
exact float64 values of the rounded tensors. Workloads with N_q queries
against N_k keys draw Q as [B, H, N_q, d] and K, V as [B, H, N_k, d] the same
way (dO, if any, as [B, H, N_q, d]); a causal workload only differs in the
mask the computation applies, not in its inputs.
"""

from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "fp32" or "bf16"
    seed: int
    q_std: float = 1.0
    backward: bool = False
    n_k: int | None = None   # keys per head (None: N, self-attention shape)
    causal: bool = False

    @property
    def Nq(self) -> int:
        return self.N

    @property
    def Nk(self) -> int:
        return self.N if self.n_k is None else self.n_k

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def kv_shape(self):
        return (self.B, self.H, self.Nk, self.d)

    def with_size(self, B=None, H=None, N=None, n_k=None):
        return dataclasses.replace(self, B=B or self.B, H=H or self.H, N=N or self.N,
                                   n_k=n_k or self.n_k)


WORKLOADS = [
    Workload("single_head_fp32_b1h1_n256_d64", 1, 1, 256, 64, "fp32", seed=1),
    Workload("mha_bf16_b4h8_n1024_d64", 4, 8, 1024, 64, "bf16", seed=2),
    Workload("mha_bf16_b2h16_n4096_d128", 2, 16, 4096, 128, "bf16", seed=3),
    Workload("long_bf16_b1h16_n16384_d128_qstd3", 1, 16, 16384, 128, "bf16", seed=4, q_std=3.0),
    Workload("fwdbwd_bf16_b2h16_n4096_d128", 2, 16, 4096, 128, "bf16", seed=5, backward=True),
]
# Workloads of the masked and unequal-length paths: causal attention at the
# headline shape; one device's query shard (N_q = 2048 of a 16384-long
# sequence split over 8 devices) against the whole key sequence, with the
# long workload's spread of scores; and decoding (one new query per
# sequence against an 8192-key history).
EXTRA_WORKLOADS = [
    Workload("causal_bf16_b2h16_n4096_d128", 2, 16, 4096, 128, "bf16", seed=6, causal=True),
    Workload("shard_bf16_b1h16_nq2048_nk16384_d128_qstd3", 1, 16, 2048, 128, "bf16", seed=7,
             q_std=3.0, n_k=16384),
    Workload("decode_bf16_b8h16_nq1_nk8192_d128", 8, 16, 1, 128, "bf16", seed=8, n_k=8192),
]
BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}
HEADLINE = WORKLOADS[2]


def make_inputs(w: Workload, with_grad_output: bool | None = None):
    """CPU tensors q, k, v (and do) for workload `w`, drawn from its seed."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    shape = w.shape()
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(w.kv_shape(), generator=g, dtype=torch.float32)
    v = torch.randn(w.kv_shape(), generator=g, dtype=torch.float32)
    out = {"q": q * w.q_std, "k": k, "v": v}
    if with_grad_output if with_grad_output is not None else w.backward:
        out["do"] = torch.randn(shape, generator=g, dtype=torch.float32)
    return {name: t.to(w.torch_dtype).contiguous() for name, t in out.items()}


def to_f64(t):
    """Exact float64 NumPy copy of a (CPU or device) tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
