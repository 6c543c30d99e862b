"""The seeded input recipe: shapes, dtypes, determinism and distributions."""

import torch

from tiled_attention_17_amd.workloads import EXTRA_WORKLOADS, WORKLOADS, BY_NAME, HEADLINE, make_inputs


def test_table():
    assert [w.N for w in WORKLOADS] == [256, 1024, 4096, 16384, 4096]
    assert [w.d for w in WORKLOADS] == [64, 64, 128, 128, 128]
    assert WORKLOADS[0].dtype == "fp32" and all(w.dtype == "bf16" for w in WORKLOADS[1:])
    assert HEADLINE.name == "mha_bf16_b2h16_n4096_d128"
    assert WORKLOADS[4].backward and not any(w.backward for w in WORKLOADS[:4])
    assert abs(HEADLINE.scale - 128 ** -0.5) < 1e-15


def test_deterministic_and_shaped():
    w = BY_NAME["mha_bf16_b4h8_n1024_d64"].with_size(B=1, H=2, N=128)
    a, b = make_inputs(w), make_inputs(w)
    for name in ("q", "k", "v"):
        assert a[name].shape == (1, 2, 128, 64) and a[name].dtype == torch.bfloat16
        assert a[name].is_contiguous()
        assert torch.equal(a[name], b[name])
    assert "do" not in a


def test_backward_has_grad_output_and_q_std():
    w = WORKLOADS[4].with_size(B=1, H=1, N=512)
    x = make_inputs(w)
    assert set(x) == {"q", "k", "v", "do"}
    w4 = WORKLOADS[3].with_size(B=1, H=2, N=2048)
    y = make_inputs(w4)
    assert 2.8 < y["q"].float().std().item() < 3.2
    assert 0.9 < y["k"].float().std().item() < 1.1


def test_bf16_is_rne_of_fp32_draw():
    w = WORKLOADS[1].with_size(B=1, H=1, N=64)
    g = torch.Generator().manual_seed(w.seed)
    q32 = torch.randn(w.shape(), generator=g)
    assert torch.equal(make_inputs(w)["q"], q32.to(torch.bfloat16))


def test_unequal_lengths_and_causal_workloads():
    causal, shard, decode = EXTRA_WORKLOADS
    assert causal.causal and causal.shape() == HEADLINE.shape() and causal.Nk == causal.N
    assert (shard.Nq, shard.Nk, shard.q_std) == (2048, 16384, 3.0)
    assert (decode.B, decode.H, decode.Nq, decode.Nk) == (8, 16, 1, 8192)
    x = make_inputs(shard.with_size(H=2, N=64, n_k=200))
    assert x["q"].shape == (1, 2, 64, 128) and x["k"].shape == (1, 2, 200, 128)
    assert x["v"].shape == x["k"].shape
    y = make_inputs(shard.with_size(H=2, N=64, n_k=200), with_grad_output=True)
    assert y["do"].shape == (1, 2, 64, 128) and torch.equal(x["q"], y["q"])
