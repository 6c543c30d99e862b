"""GPU check of attn_bwd_ex_noalloc, the backward entry point that allocates nothing.

Two calls in a row through the C ABI, the second with a smaller input (so it
reads the fixed scratch array the first call left filled), each against
attn_bwd_ex on the same inputs with a workspace of its own: the two run the
same kernels on the same row terms, so the gradients must agree bit for bit,
which is inside the bf16 bar (max abs error <= 2e-2) the parity tests hold
attn_bwd_ex to against the float64 oracle. Then the same entry point under HIP
graph capture (beside a key-split forward given its workspace), replayed three
times against the eager results.
"""

import pytest

torch = pytest.importorskip("torch")

import tiled_attention_17_amd as ta  # noqa: E402
from tiled_attention_17_amd.workloads import Workload, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ta.library()


def _run(w, causal):
    x = {k: t.cuda() for k, t in make_inputs(w, with_grad_output=True).items()}
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    ref = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=causal)
    got = [torch.full_like(t, float("nan")) for t in ref]
    ta.attn_bwd_ex_noalloc(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=causal,
                           dq=got[0], dk=got[1], dv=got[2])
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{w.name} {name}: max diff {(a.float() - b.float()).abs().max().item():.3e}"


def test_noalloc_backward_two_calls_second_smaller():
    big = Workload("noalloc_b2h3_nq700_nk900_d128_causal", 2, 3, 700, 128, "bf16", seed=71, n_k=900)
    small = Workload("noalloc_b1h2_nq200_nk150_d64", 1, 2, 200, 64, "bf16", seed=72, n_k=150, q_std=3.0)
    _run(big, causal=True)
    _run(small, causal=False)


def test_noalloc_backward_under_graph_capture():
    # The callers this entry point is for include code under HIP graph capture:
    # a graph holding a key-split forward (workspace given) and the
    # allocation-free backward replays to the eager results, bit for bit, three
    # times, with eager work and synchronisations between the replays.
    w = Workload("noalloc_graph_b1h2_nq300_nk260_d128_causal", 1, 2, 300, 128, "bf16", seed=73, n_k=260)
    x = {k: t.cuda() for k, t in make_inputs(w, with_grad_output=True).items()}
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o_ref, lse_ref = ta.attn_fwd_ex(q, k, v, w.scale, causal=True, num_splits=2)
    g_ref = ta.attn_bwd_ex(q, k, v, o_ref, do, lse_ref, w.scale, causal=True)
    ws = torch.empty(ta.attn_fwd_ex_workspace_bytes(1, 2, 300, 260, 128, 2), dtype=torch.uint8, device="cuda")
    o, lse = torch.empty_like(o_ref), torch.empty_like(lse_ref)
    grads = [torch.empty_like(t) for t in g_ref]

    def step():
        ta.attn_fwd_ex(q, k, v, w.scale, causal=True, num_splits=2, out=o, lse=lse, workspace=ws)
        ta.attn_bwd_ex_noalloc(q, k, v, o, do, lse, w.scale, causal=True, dq=grads[0], dk=grads[1], dv=grads[2])

    step()  # eager once first (the library looks up its per-device state here, not under capture)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        for t in [o, lse] + grads:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        for name, a, b in zip(("dQ", "dK", "dV"), grads, g_ref):
            assert torch.equal(a, b), f"{name}: max diff {(a.float() - b.float()).abs().max().item():.3e}"

