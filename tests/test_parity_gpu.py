"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Bars, stated by the workload specification: bf16 inputs -> max abs error
<= 2e-2 on O, dQ, dK, dV; fp32 inputs -> <= 1e-5 on O; LSE -> <= 1e-3 (abs).
Because gradients of the large workloads are small in magnitude (|dV| ~ 0.1),
every bf16 comparison also bounds the error relative to the largest
reference magnitude (2e-2), so that a wrongly scaled or missing result cannot
pass on the absolute bar alone.

The oracle always receives the exact float64 values of the (bf16-rounded)
inputs the GPU saw, so the comparison measures kernel error, not input
rounding.
"""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import tiled_attention_17_amd as ta  # noqa: E402
from oracle import attention_forward  # noqa: E402
from oracle_pool import backward_all, forward_all  # noqa: E402
from tiled_attention_17_amd.workloads import WORKLOADS, Workload, make_inputs, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
BF16_REL = 2e-2
FP32_TOL = 1e-5
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ta.library()  # fail loudly if the HIP library is missing


def _cuda(x):
    return {k: t.cuda() for k, t in x.items()}


def _max_err(got, want):
    return float(np.max(np.abs(got - want))) if want.size else 0.0


def _assert_close(name, got, want, tol, rel=None):
    err = _max_err(got, want)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert err <= tol, f"{name}: max abs err {err:.3e} > {tol:.1e}"
    if rel is not None and want.size:
        scale = float(np.max(np.abs(want)))
        assert err <= rel * scale + 1e-6, f"{name}: max err {err:.3e} > {rel} * max|ref| {scale:.3e}"


def _check_fwd(x, o, lse, scale, tol, rel, rows=None, heads=None):
    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    o, lse = to_f64(o), to_f64(lse)
    heads = heads if heads is not None else list(np.ndindex(*q.shape[:2]))
    for (b, h) in heads:
        qi = q[b, h] if rows is None else q[b, h][rows]
        ro, rl = attention_forward(qi, k[b, h], v[b, h], scale)
        go = o[b, h] if rows is None else o[b, h][rows]
        gl = lse[b, h] if rows is None else lse[b, h][rows]
        _assert_close(f"O[{b},{h}]", go, ro, tol, rel)
        _assert_close(f"LSE[{b},{h}]", gl, rl, LSE_TOL)


def _wl(B, H, N, d, dtype="bf16", seed=0, q_std=1.0):
    return Workload(f"t_{B}_{H}_{N}_{d}_{dtype}", B, H, N, d, dtype, seed=seed, q_std=q_std)


# ---------------------------------------------------------------------------
# small sizes: several tiles and ragged tails, every tile configuration
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 2, 64), (2, 3, 200), (1, 1, 1), (1, 2, 37), (2, 2, 513),
                                   (1, 2, 1000), (1, 1, 2048)])
def test_fwd_bf16_small(B, H, N, d):
    w = _wl(B, H, N, d, seed=N + d)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    _check_fwd(x, o, lse, w.scale, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("waves", ["2", "4", "8"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_bf16_tile_configs(waves, d, monkeypatch):
    monkeypatch.setenv("TILED_ATTN_FWD_WAVES", waves)
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT", "1")
    w = _wl(2, 2, 777, d, seed=5, q_std=3.0)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    _check_fwd(x, o, lse, w.scale, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_running_max_jumps(d, causal, monkeypatch):
    # Key rows grow in steps along the sequence, so each row's scores jump far
    # above the running max mid-sweep: by ~20 (base 2) at key 448 (mid-tile,
    # in a 32-key block after others of the same tile), by ~70 at key 640 and
    # by more than fp32's exponent range at key 800 (2^x overflows before the
    # max is moved). The 256-query ping-pong kernel is forced, whose unmasked
    # tiles skip the row max until a block's sum shows such a jump.
    monkeypatch.setenv("TILED_ATTN_FWD_WAVES", "8")
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT", "1")
    w = _wl(1, 2, 1000, d, seed=77)
    x = make_inputs(w)
    mult = torch.ones(w.N)
    mult[448:] = 6.0
    mult[640:] = 20.0
    mult[800:] = 60.0
    x["k"] = (x["k"].float() * mult[None, None, :, None]).to(torch.bfloat16).contiguous()
    x = _cuda(x)
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    torch.cuda.synchronize()
    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    ro, rl = attention_forward(q, k, v, w.scale, causal=causal)
    assert float(np.max(rl)) * np.log2(np.e) > 128 + 20  # the last jump passes fp32's range
    _assert_close("O", to_f64(o), ro, BF16_TOL, BF16_REL)
    _assert_close("LSE", to_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("waves", ["2", "4"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 37, 64, 100, 200, 257, 777, 1000])
def test_fwd_bf16_keys_split_in_workgroup(N, d, waves, monkeypatch):
    # Two wave groups take the two halves of the key tiles and merge through
    # LDS: odd tile counts (group 1 idles one step), a ragged last tile, and
    # N below two tiles (group 1 sees no key) all go through the merge.
    monkeypatch.setenv("TILED_ATTN_FWD_WAVES", waves)
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT", "2")
    w = _wl(2, 3, N, d, seed=400 + N + d, q_std=3.0)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    _check_fwd(x, o, lse, w.scale, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 31, 100, 256, 300])
def test_fwd_fp32_small(N, d):
    w = _wl(1, 2, N, d, dtype="fp32", seed=N)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    _check_fwd(x, o, lse, w.scale, FP32_TOL, None)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 2, 64), (1, 1, 1), (2, 2, 200), (1, 2, 513), (1, 1, 1024)])
def test_bwd_bf16_small(B, H, N, d):
    w = _wl(B, H, N, d, seed=1000 + N + d)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    dq, dk, dv = ta.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale)
    torch.cuda.synchronize()
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    rq, rk, rv = backward_all(q, k, v, to_f64(o), do, w.scale)
    _assert_close("dQ", to_f64(dq), rq, BF16_TOL, BF16_REL)
    _assert_close("dK", to_f64(dk), rk, BF16_TOL, BF16_REL)
    _assert_close("dV", to_f64(dv), rv, BF16_TOL, BF16_REL)


# ---------------------------------------------------------------------------
# full-size workloads in the benchmark's launch configuration, whole outputs
# ---------------------------------------------------------------------------

def _check_all(name, go, gl, ro, rl, tol, rel):
    """Every element of O and LSE, reported per head."""
    for (b, h) in np.ndindex(*ro.shape[:2]):
        _assert_close(f"{name} O[{b},{h}]", go[b, h], ro[b, h], tol, rel)
        _assert_close(f"{name} LSE[{b},{h}]", gl[b, h], rl[b, h], LSE_TOL)


def test_workload_fp32_single_head_full():
    w = WORKLOADS[0]
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    _check_fwd(x, o, lse, w.scale, FP32_TOL, None)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("idx", [1, 2])
def test_workload_bf16_full_every_head(idx):
    # B=4 H=8 N=1024 d=64 and the headline B=2 H=16 N=4096 d=128: every
    # element of O and LSE against the oracle.
    w = WORKLOADS[idx]
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    ro, rl = forward_all(q, k, v, w.scale)
    _check_all(w.name, to_f64(o), to_f64(lse), ro, rl, BF16_TOL, BF16_REL)


@pytest.mark.timeout(900)
def test_workload_long_sequence_every_row():
    # B=1 H=16 N=16384 d=128, Q ~ N(0, 3^2): all 16 x 16384 rows, the oracle
    # taken in blocks of 1024 query rows against all keys.
    w = WORKLOADS[3]
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    ro, rl = forward_all(q, k, v, w.scale, row_block=1024)
    _check_all(w.name, to_f64(o), to_f64(lse), ro, rl, BF16_TOL, BF16_REL)


@pytest.mark.timeout(900)
def test_workload_fwd_bwd_every_head():
    # B=2 H=16 N=4096 d=128 forward and backward: every element of O, LSE,
    # dQ, dK and dV against the oracle.
    w = WORKLOADS[4]
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    dq, dk, dv = ta.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale)
    torch.cuda.synchronize()
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ro, rl = forward_all(q, k, v, w.scale)
    _check_all(w.name, to_f64(o), to_f64(lse), ro, rl, BF16_TOL, BF16_REL)
    ref = backward_all(q, k, v, to_f64(o), do, w.scale)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        got = to_f64(got)
        for (b, h) in np.ndindex(w.B, w.H):
            _assert_close(f"{name}[{b},{h}]", got[b, h], want[b, h], BF16_TOL, BF16_REL)


# ---------------------------------------------------------------------------
# degenerate cases, determinism, streams
# ---------------------------------------------------------------------------

def test_constant_keys_give_mean_of_values():
    w = _wl(1, 2, 300, 128, seed=8)
    x = make_inputs(w, with_grad_output=True)
    x["k"] = x["k"][:, :, :1].expand_as(x["k"]).contiguous()
    x = _cuda(x)
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    dq, dk, dv = ta.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale)
    torch.cuda.synchronize()
    v = to_f64(x["v"])
    np.testing.assert_allclose(to_f64(o), np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape),
                               atol=BF16_TOL)
    want_lse = w.scale * np.einsum("bhnd,bhd->bhn", to_f64(x["q"]), to_f64(x["k"])[:, :, 0]) + np.log(w.N)
    np.testing.assert_allclose(to_f64(lse), want_lse, atol=LSE_TOL)
    assert float(np.max(np.abs(to_f64(dq)))) <= BF16_TOL  # dQ = 0 exactly in exact arithmetic
    do = to_f64(x["do"])
    np.testing.assert_allclose(to_f64(dv), np.broadcast_to(do.mean(axis=2, keepdims=True), do.shape),
                               atol=BF16_TOL)


def test_scale_zero_is_uniform():
    w = _wl(1, 1, 130, 64, seed=9)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], 0.0)
    torch.cuda.synchronize()
    v = to_f64(x["v"])
    np.testing.assert_allclose(to_f64(o), np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape),
                               atol=BF16_TOL)
    np.testing.assert_allclose(to_f64(lse), np.log(130), atol=LSE_TOL)


def test_single_key_gradients():
    w = _wl(1, 1, 1, 128, seed=10)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    dq, dk, dv = ta.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, x["v"])
    assert torch.equal(dv, x["do"])
    assert float(dq.abs().max()) <= 1e-4 and float(dk.abs().max()) <= 1e-4


def test_empty_problem_is_noop():
    z = torch.empty(0, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = ta.attn_fwd(z, z.clone(), z.clone())
    assert o.shape == z.shape and lse.shape == (0, 2, 64)


def test_forward_and_backward_are_deterministic():
    w = _wl(2, 4, 1000, 128, seed=12)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o1, l1 = ta.attn_fwd(x["q"], x["k"], x["v"])
    o2, l2 = ta.attn_fwd(x["q"], x["k"], x["v"])
    g1 = ta.attn_bwd(x["q"], x["k"], x["v"], o1, x["do"], l1)
    g2 = ta.attn_bwd(x["q"], x["k"], x["v"], o1, x["do"], l1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_side_stream_matches_default_stream():
    w = _wl(1, 4, 700, 64, seed=13)
    x = _cuda(make_inputs(w))
    o1, l1 = ta.attn_fwd(x["q"], x["k"], x["v"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = ta.attn_fwd(x["q"], x["k"], x["v"])
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_misaligned_view_is_rejected():
    base = torch.zeros(1 * 1 * 64 * 64 + 1, dtype=torch.bfloat16, device="cuda")
    q = base[1:].view(1, 1, 64, 64)  # 2-byte offset: contiguous but not 16-byte aligned
    k = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ta.AttnError, match="aligned"):
        ta.attn_fwd(q, k, k.clone())
