"""GPU parity of the extended forward (causal mask, N_q != N_k, key splits) and the merge.

Everything goes through the C ABI (attn_fwd_ex, attn_merge) and is compared
with the float64 CPU oracle on the same inputs: attention_forward with the
causal reading query i sees key j iff j <= i + N_k - N_q, and merge_partials.
Bars as for the plain forward: bf16 -> max abs error <= 2e-2 on O (and
<= 2e-2 of the largest reference magnitude), fp32 -> <= 1e-5, LSE <= 1e-3
absolute. Rows that see no key must come back as exactly O = 0, LSE = -inf.
"""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import tiled_attention_17_amd as ta  # noqa: E402
from oracle import attention_forward, merge_partials  # noqa: E402
from oracle_pool import backward_all, forward_all  # noqa: E402
from tiled_attention_17_amd.workloads import EXTRA_WORKLOADS, Workload, make_inputs, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
BF16_REL = 2e-2
FP32_TOL = 1e-5
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ta.library()


def _cuda(x):
    return {k: t.cuda() for k, t in x.items()}


def _wl(B, H, Nq, Nk, d, dtype="bf16", seed=0, q_std=1.0, causal=False):
    return Workload(f"t_{B}_{H}_{Nq}_{Nk}_{d}_{dtype}", B, H, Nq, d, dtype, seed=seed, q_std=q_std,
                    n_k=Nk, causal=causal)


BF16_U = 2.0 ** -8  # unit roundoff of bf16 round-to-nearest-even (8 significant bits)


def _assert_grad(name, got, want):
    """A gradient (against the oracle at the given O, oracle_pool's
    backward_given_o) within 2e-2 + 2u max|ref| (one u for the rounding of the
    result to bf16, one for the bf16 rounding of the P and dS operands), and
    within 2e-2 max|ref| + 1e-4 (a wrongly scaled result fails). Needed where
    gradients grow past ~2: under the mask with N_q > N_k the first visible
    query sees one key with P = 1, and that key's dV sums dO rows with
    weights 1, 1/2, 1/3, ..."""
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    if not want.size:
        return
    err = float(np.max(np.abs(got - want)))
    scale = float(np.max(np.abs(want)))
    bound = BF16_TOL + 2 * BF16_U * scale
    assert err <= bound, f"{name}: max abs err {err:.3e} > {bound:.3e} (max|ref| {scale:.3e})"
    assert err <= BF16_REL * scale + 1e-4, f"{name}: max err {err:.3e} > {BF16_REL} * max|ref| {scale:.3e} + 1e-4"


def _assert_o(name, got, want, tol, rel):
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= tol, f"{name}: max abs err {err:.3e} > {tol:.1e}"
    if rel is not None and want.size:
        scale = float(np.max(np.abs(want)))
        assert err <= rel * scale + 1e-6, f"{name}: max err {err:.3e} > {rel} * max|ref| {scale:.3e}"


def _assert_lse(name, got, want):
    empty = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), empty), f"{name}: rows without keys differ"
    if (~empty).any():
        err = float(np.max(np.abs(got[~empty] - want[~empty])))
        assert err <= LSE_TOL, f"{name}: max abs err {err:.3e} > {LSE_TOL:.1e}"


def _check(x, o, lse, scale, causal, tol, rel, heads=None, rows=None):
    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    o, lse = to_f64(o), to_f64(lse)
    heads = heads if heads is not None else list(np.ndindex(*q.shape[:2]))
    for (b, h) in heads:
        ro, rl = attention_forward(q[b, h], k[b, h], v[b, h], scale, causal=causal)
        go, gl = o[b, h], lse[b, h]
        if rows is not None:
            ro, rl, go, gl = ro[rows], rl[rows], go[rows], gl[rows]
        empty = np.isneginf(rl)
        assert np.all(go[empty] == 0), f"O[{b},{h}]: rows without keys are not 0"
        _assert_o(f"O[{b},{h}]", go, ro, tol, rel)
        _assert_lse(f"LSE[{b},{h}]", gl, rl)


# ---------------------------------------------------------------------------
# causal, equal lengths: every tile configuration, ragged N, both dtypes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("waves", ["2", "4", "8"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 70, 256, 777, 1100])
def test_causal_bf16_tile_configs(N, d, waves, monkeypatch):
    monkeypatch.setenv("TILED_ATTN_FWD_WAVES", waves)
    w = _wl(1, 3, N, N, d, seed=N + d, q_std=2.0, causal=True)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, True, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 33, 200])
def test_causal_fp32(N, d):
    w = _wl(1, 2, N, N, d, dtype="fp32", seed=N, causal=True)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, True, FP32_TOL, None)


@pytest.mark.parametrize("ksplit", ["1", "2", "2/32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (37, 37), (64, 64), (100, 100), (257, 257), (777, 777),
                                   (150, 90), (40, 1000)])
def test_fp32_keys_split_in_workgroup(Nq, Nk, d, causal, ksplit, monkeypatch):
    # fp32 forward with a workgroup's key tiles dealt out to its waves and
    # merged through LDS (2; at d = 64 and these grid sizes the 16-query
    # 16x16x4 kernel, and "2/32" the 32-query one) and with one key loop per
    # wave (1): fewer tiles than waves (waves without a key), tile counts not
    # a multiple of the waves, a ragged last tile, N_q != N_k (rows without a
    # visible key under the mask) and a large query spread.
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT", ksplit.split("/")[0])
    if ksplit == "2/32":
        monkeypatch.setenv("TILED_ATTN_FWD_F32_BM", "32")
    w = _wl(1, 2, Nq, Nk, d, dtype="fp32", seed=600 + Nq + Nk + d, q_std=3.0, causal=causal)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, causal, FP32_TOL, None)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("ksplit", ["1", "2"])
def test_fp32_keys_split_in_workgroup_with_key_splits(ksplit, d, monkeypatch):
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT", ksplit)
    w = _wl(2, 1, 70, 1500, d, dtype="fp32", seed=610)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True, num_splits=3)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, True, FP32_TOL, None)


def test_causal_first_row_is_first_value():
    w = _wl(2, 2, 300, 300, 128, seed=3, causal=True)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0], x["v"][:, :, 0])
    want = w.scale * (x["q"][:, :, 0].double() * x["k"][:, :, 0].double()).sum(-1)
    assert float((lse[:, :, 0].double() - want).abs().max()) <= 1e-5


def test_causal_ignores_hidden_keys():
    # Keys and values no query may see (all keys after the last query's
    # window do not exist with equal lengths, so use N_q < N_k and perturb the
    # keys hidden from the first half of the queries).
    w = _wl(1, 2, 256, 512, 64, seed=4, causal=True)
    x = _cuda(make_inputs(w))
    o1, l1 = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True)
    k2, v2 = x["k"].clone(), x["v"].clone()
    first_hidden = 128 + 512 - 256  # first key hidden from query 127
    k2[:, :, first_hidden:] = 40.0
    v2[:, :, first_hidden:] = -7.0
    o2, l2 = ta.attn_fwd_ex(x["q"], k2, v2, w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :128], o2[:, :, :128]) and torch.equal(l1[:, :, :128], l2[:, :, :128])


# ---------------------------------------------------------------------------
# N_q != N_k, with and without the mask (N_q > N_k leaves rows with no key)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("bn", ["64", "128"])
@pytest.mark.parametrize("waves", ["2", "4"])
@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 2, 100, 1000), (2, 1, 257, 1024), (1, 1, 64, 1500), (1, 2, 300, 129),
                                       (1, 1, 2, 2048), (1, 3, 513, 4100)])
def test_keys_split_tile_sizes_d64(B, H, Nq, Nk, waves, bn, monkeypatch):
    # The bf16 key split at d = 64 with 64- and 128-key tiles (the launch
    # picks 128 for large grids of long key ranges), ragged key ends included.
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT", "2")
    monkeypatch.setenv("TILED_ATTN_FWD_WAVES", waves)
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT_BN", bn)
    w = _wl(B, H, Nq, Nk, 64, seed=70 + Nq + Nk)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, False, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("waves,ksplit", [("2", "1"), ("4", "1"), ("8", "1"), ("2", "2"), ("4", "2")])
@pytest.mark.parametrize("Nq,Nk", [(1, 1000), (100, 700), (300, 129), (513, 64), (64, 2048)])
def test_unequal_lengths_bf16(Nq, Nk, waves, ksplit, causal, monkeypatch):
    # ksplit "2": the keys of a workgroup split between two wave groups
    # (unmasked launches only; the causal cases take the other kernels)
    monkeypatch.setenv("TILED_ATTN_FWD_WAVES", waves)
    monkeypatch.setenv("TILED_ATTN_FWD_KSPLIT", ksplit)
    w = _wl(2, 2, Nq, Nk, 128, seed=Nq + Nk, q_std=3.0)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, causal, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("causal", [False, True])
def test_unequal_lengths_d64_and_fp32(causal):
    w = _wl(1, 2, 150, 400, 64, seed=11)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    wf = _wl(1, 2, 150, 90, 64, dtype="fp32", seed=12)
    xf = _cuda(make_inputs(wf))
    of, lf = ta.attn_fwd_ex(xf["q"], xf["k"], xf["v"], wf.scale, causal=causal)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, causal, BF16_TOL, BF16_REL)
    _check(xf, of, lf, wf.scale, causal, FP32_TOL, None)


def test_no_keys_gives_empty_rows():
    q = torch.randn(1, 2, 70, 64, device="cuda").to(torch.bfloat16)
    kv = torch.empty(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = ta.attn_fwd_ex(q, kv, kv.clone())
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


# ---------------------------------------------------------------------------
# key splits (partials in the workspace, then the merge kernel)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("waves", ["2", "4", "8"])
def test_splits_bf16(splits, waves, causal, monkeypatch):
    monkeypatch.setenv("TILED_ATTN_FWD_WAVES", waves)
    w = _wl(1, 2, 300, 1000, 128, seed=20 + splits, q_std=2.0)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal, num_splits=splits)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, causal, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("causal", [False, True])
def test_splits_fp32_and_d64(causal):
    w = _wl(1, 2, 40, 500, 64, dtype="fp32", seed=30)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal, num_splits=3)
    wb = _wl(2, 1, 200, 300, 64, seed=31)
    xb = _cuda(make_inputs(wb))
    ob, lb = ta.attn_fwd_ex(xb["q"], xb["k"], xb["v"], wb.scale, causal=causal, num_splits=5)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, causal, FP32_TOL, None)
    _check(xb, ob, lb, wb.scale, causal, BF16_TOL, BF16_REL)


def test_splits_match_single_pass_closely():
    # Same inputs, one pass vs four splits: both within the bar of the
    # oracle, and of each other (fp32 partials, one rounding at the end).
    w = _wl(2, 2, 64, 4096, 128, seed=40)
    x = _cuda(make_inputs(w))
    o1, l1 = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=1)
    o4, l4 = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=4)
    torch.cuda.synchronize()
    assert float((o1.float() - o4.float()).abs().max()) <= 2 * BF16_TOL
    assert float((l1 - l4).abs().max()) <= LSE_TOL
    _check(x, o4, l4, w.scale, False, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("decode", ["0", "1"])
@pytest.mark.parametrize("splits", [1, 3, 0])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nk", [1, 7, 65, 300, 4096])
def test_one_query_per_head(Nk, d, splits, decode, monkeypatch):
    # N_q = 1 on the one-query kernel (0) and on the tiled kernels (1): a
    # ragged last key block, fewer key blocks than waves (waves without a
    # key), key splits given and chosen by the library.
    monkeypatch.setenv("TILED_ATTN_FWD_DECODE", decode)
    w = _wl(2, 3, 1, Nk, d, seed=700 + Nk + d, q_std=3.0)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=splits)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, False, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("Nk", [1, 130, 2000])
def test_one_query_per_head_causal_and_empty(Nk):
    # With one query the causal window covers every key; and a head without
    # keys gives O = 0, LSE = -inf.
    w = _wl(3, 2, 1, Nk, 128, seed=710 + Nk)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, True, BF16_TOL, BF16_REL)
    kv = torch.empty(3, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    o0, l0 = ta.attn_fwd_ex(x["q"], kv, kv.clone())
    torch.cuda.synchronize()
    assert torch.all(o0 == 0) and torch.all(torch.isneginf(l0))


def test_auto_splits_decode_shape():
    w = _wl(4, 8, 1, 3000, 128, seed=41)
    x = _cuda(make_inputs(w))
    s = ta.attn_fwd_ex_auto_splits(w.B, w.H, 1, 3000, 128)
    assert s > 1
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=0)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, False, BF16_TOL, BF16_REL)


def test_more_splits_than_key_tiles():
    w = _wl(1, 1, 10, 200, 64, seed=42)
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=16)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, False, BF16_TOL, BF16_REL)


# ---------------------------------------------------------------------------
# attn_merge on its own
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp32"])
def test_merge_against_oracle(d, out_dtype):
    rng = np.random.default_rng(d)
    P, B, H, N = 5, 2, 3, 77
    o_parts = rng.standard_normal((P, B, H, N, d))
    lse_parts = rng.standard_normal((P, B, H, N)) * 4.0 + 30.0
    lse_parts[1, 0, 0] = -np.inf                 # an empty part
    lse_parts[:, 1, 2, :5] = -np.inf             # rows whose parts are all empty
    o_parts[:, 1, 2, :5] = 0.0
    o_parts = o_parts.astype(np.float32)
    lse_parts = lse_parts.astype(np.float32)
    dt = torch.float32 if out_dtype == "fp32" else torch.bfloat16
    o, lse = ta.attn_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(), dtype=dt)
    torch.cuda.synchronize()
    ro, rl = merge_partials(o_parts.astype(np.float64), lse_parts.astype(np.float64))
    go, gl = to_f64(o), to_f64(lse)
    _assert_o("O", go, ro, FP32_TOL if out_dtype == "fp32" else BF16_TOL, None)
    _assert_lse("LSE", gl, rl)
    assert np.all(go[1, 2, :5] == 0)


def test_merge_of_gpu_key_ranges_equals_whole():
    # Sequence-split use: attention of one query block over two halves of the
    # keys (each on the GPU, fp32 inputs for an fp32 comparison), merged on
    # the GPU, against the oracle over all keys.
    w = _wl(1, 2, 96, 600, 64, dtype="fp32", seed=50)
    x = _cuda(make_inputs(w))
    parts = [ta.attn_fwd_ex(x["q"], x["k"][:, :, a:b].contiguous(), x["v"][:, :, a:b].contiguous(), w.scale)
             for a, b in ((0, 250), (250, 600))]
    o_parts = torch.stack([p[0] for p in parts]).contiguous()
    lse_parts = torch.stack([p[1] for p in parts]).contiguous()
    o, lse = ta.attn_merge(o_parts, lse_parts, dtype=torch.float32)
    torch.cuda.synchronize()
    _check(x, o, lse, w.scale, False, FP32_TOL, None)


# ---------------------------------------------------------------------------
# attn_fwd_ex_timed: attn_fwd_ex's results, and events around its attention
# kernel alone
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,B,H,Nq,Nk,d,causal,splits,waves", [
    ("bf16", 1, 2, 1000, 1000, 128, False, 1, "8"),  # ping-pong kernel, ragged tail
    ("bf16", 1, 4, 1024, 1024, 64, False, 1, None),  # keys split between the wave groups
    ("bf16", 1, 2, 700, 700, 64, True, 3, "4"),      # mask, key splits and the merge
    ("bf16", 2, 2, 1, 2000, 128, False, 0, None),    # one query per head, split, merged
    ("fp32", 1, 1, 256, 256, 64, False, 1, None),    # 16-query fp32 kernel
    ("fp32", 1, 2, 130, 300, 128, True, 2, None),    # fp32 with the mask, split, merged
])
def test_fwd_ex_timed(dtype, B, H, Nq, Nk, d, causal, splits, waves, monkeypatch):
    if waves is not None:
        monkeypatch.setenv("TILED_ATTN_FWD_WAVES", waves)
    w = _wl(B, H, Nq, Nk, d, dtype=dtype, seed=60 + Nq % 7, causal=causal)
    x = _cuda(make_inputs(w))
    o1, lse1 = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal, num_splits=splits)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    outer0, outer1, start, stop = ev(), ev(), ev(), ev()
    outer0.record()
    o2, lse2 = ta.attn_fwd_ex_timed(x["q"], x["k"], x["v"], start, stop, w.scale, causal=causal,
                                    num_splits=splits)
    outer1.record()
    o3, lse3 = ta.attn_fwd_ex_timed(x["q"], x["k"], x["v"], None, None, w.scale, causal=causal,
                                    num_splits=splits)
    torch.cuda.synchronize()
    # Same kernels on the same inputs: bitwise the same results.
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    assert torch.equal(o1, o3) and torch.equal(lse1, lse3)
    tol, rel = (FP32_TOL, None) if dtype == "fp32" else (BF16_TOL, BF16_REL)
    _check(x, o2, lse2, w.scale, causal, tol, rel)
    inner, outer = start.elapsed_time(stop), outer0.elapsed_time(outer1)
    assert 0.0 < inner <= outer + 1e-3, (inner, outer)


@pytest.mark.parametrize("d", [64, 128])
def test_auto_plan_splits_the_last_round(d):
    # 288 heads of 256 queries: one whole round of 256-query workgroups on a
    # 256-CU device and 32 heads over. With num_splits = 0 the library runs
    # the first 256 heads unsplit and splits the keys of the other 32 (two
    # attention launches and a merge).
    w = _wl(1, 288, 256, 1024, d, seed=80 + d)
    x = _cuda(make_inputs(w))
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert ta.attn_fwd_ex_workspace_bytes(1, 288, 256, 1024, d, 0) == 2 * 32 * 256 * (d + 1) * 4
    o0, l0 = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=0)
    o1, l1 = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=1)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    o2, l2 = ta.attn_fwd_ex_timed(x["q"], x["k"], x["v"], start, stop, w.scale, num_splits=0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o2) and torch.equal(l0, l2)
    assert start.elapsed_time(stop) > 0.0
    # The heads of the whole round run the one-pass kernel on the same tiles.
    assert torch.equal(o0[:, :256], o1[:, :256]) and torch.equal(l0[:, :256], l1[:, :256])
    _check_whole(x, o0, l0, w.scale, False)


# ---------------------------------------------------------------------------
# full-size workloads of these paths, whole outputs
# ---------------------------------------------------------------------------

def _check_whole(x, o, lse, scale, causal, row_block=None):
    """Every element of O and LSE against the oracle (evaluated in a thread pool)."""
    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    ro, rl = forward_all(q, k, v, scale, causal=causal, row_block=row_block)
    go, gl = to_f64(o), to_f64(lse)
    for (b, h) in np.ndindex(*q.shape[:2]):
        empty = np.isneginf(rl[b, h])
        assert np.all(go[b, h][empty] == 0), f"O[{b},{h}]: rows without keys are not 0"
        _assert_o(f"O[{b},{h}]", go[b, h], ro[b, h], BF16_TOL, BF16_REL)
        _assert_lse(f"LSE[{b},{h}]", gl[b, h], rl[b, h])


@pytest.mark.timeout(600)
def test_workload_causal_every_head():
    w = EXTRA_WORKLOADS[0]
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True)
    torch.cuda.synchronize()
    _check_whole(x, o, lse, w.scale, True)


@pytest.mark.timeout(600)
def test_workload_shard_every_row():
    w = EXTRA_WORKLOADS[1]
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=0)
    torch.cuda.synchronize()
    _check_whole(x, o, lse, w.scale, False, row_block=1024)


def test_workload_decode_every_head():
    w = EXTRA_WORKLOADS[2]
    x = _cuda(make_inputs(w))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, num_splits=0)
    torch.cuda.synchronize()
    _check_whole(x, o, lse, w.scale, False)


# ---------------------------------------------------------------------------
# backward with the mask and unequal lengths
# ---------------------------------------------------------------------------

def _check_bwd(x, o, dq, dk, dv, scale, causal, heads=None):
    from oracle_pool import backward_given_o
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    o = to_f64(o)
    g = [to_f64(t) for t in (dq, dk, dv)]
    heads = heads if heads is not None else list(np.ndindex(*q.shape[:2]))
    for (b, h) in heads:
        ref = backward_given_o(q[b, h], k[b, h], v[b, h], o[b, h], do[b, h], scale, causal=causal)
        for name, got, want in zip(("dQ", "dK", "dV"), g, ref):
            _assert_o(f"{name}[{b},{h}]", got[b, h], want, BF16_TOL, BF16_REL)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (64, 64), (200, 200), (513, 513), (100, 700), (700, 100),
                                   (300, 129), (1, 1000), (777, 1100), (1100, 777), (1536, 1536)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("waves", ["4", "8"])
def test_bwd_ex_small(Nq, Nk, d, causal, waves, monkeypatch):
    # Both workgroup shapes of each sweep (dK/dV: 128 keys in 4 waves or 256
    # in 8; dQ: 128 queries in 4 waves, lock-step, or 256 in 8) on every case,
    # whichever the library would pick for the shape.
    monkeypatch.setenv("TILED_ATTN_BWD_DKDV_WAVES", waves)
    monkeypatch.setenv("TILED_ATTN_BWD_DQ_WAVES", waves)
    w = _wl(1, 2, Nq, Nk, d, seed=60 + Nq + Nk + d)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    dq, dk, dv = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_bwd(x, o, dq, dk, dv, w.scale, causal)
    if causal and Nq > Nk:  # queries that see no key get dQ = 0 exactly
        assert torch.all(dq[:, :, :Nq - Nk] == 0)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ex_ignores_stale_workspace(d, causal):
    # The workspace holds the row terms D_i; its contents on entry are ignored:
    # every term the dK/dV sweep reads (also for queries that see no key, whose
    # zero P it multiplies) is written earlier in the same call. A workspace
    # full of NaN must give the same gradients, bit for bit, as a zeroed one.
    w = _wl(1, 3, 777, 300, d, seed=90 + d + causal)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    need = ta.attn_bwd_workspace_bytes(1, 3, 777, d)
    clean = torch.zeros(need, dtype=torch.uint8, device="cuda")
    stale = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN floats
    ref = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=causal, workspace=clean)
    got = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=causal, workspace=stale)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name}: max diff {(a.float() - b.float()).abs().max().item():.3e}"
    assert not torch.isnan(stale.view(torch.float32)).any()  # every row term was written


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_ex_empty_sides(d):
    q = torch.randn(1, 2, 70, d, device="cuda").to(torch.bfloat16)
    kv = torch.randn(1, 2, 90, d, device="cuda").to(torch.bfloat16)
    none_q = q[:, :, :0].contiguous()
    none_kv = kv[:, :, :0].contiguous()
    # no query: dK = dV = 0
    o0 = none_q.clone()
    lse0 = torch.empty(1, 2, 0, device="cuda")
    dq, dk, dv = ta.attn_bwd_ex(none_q, kv, kv.clone(), o0, o0.clone(), lse0)
    # no key: O = 0, LSE = -inf from the forward, dQ = 0
    o, lse = ta.attn_fwd_ex(q, none_kv, none_kv.clone())
    dq2, dk2, dv2 = ta.attn_bwd_ex(q, none_kv, none_kv.clone(), o, q.clone(), lse)
    torch.cuda.synchronize()
    assert dk.shape == kv.shape and torch.all(dk == 0) and torch.all(dv == 0)
    assert torch.all(dq2 == 0) and dk2.numel() == 0


@pytest.mark.timeout(900)
def test_workload_causal_fwd_bwd_every_head():
    # Causal attention at the forward + backward workload's shape, every head.
    w = _wl(2, 16, 4096, 4096, 128, seed=5, causal=True)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=True)
    dq, dk, dv = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=True)
    torch.cuda.synchronize()
    _check_whole(x, o, lse, w.scale, True)
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = backward_all(q, k, v, to_f64(o), do, w.scale, causal=True)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        got = to_f64(got)
        for (b, h) in np.ndindex(w.B, w.H):
            _assert_o(f"{name}[{b},{h}]", got[b, h], want[b, h], BF16_TOL, BF16_REL)


# ---------------------------------------------------------------------------
# size extremes: a long sequence and a grid of many small heads
# ---------------------------------------------------------------------------

@pytest.mark.timeout(900)
@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_fwd_bwd_whole(causal):
    # One head of 16384 queries and keys (four times the forward + backward
    # workload's length, 64 query tiles and 64 key tiles per sweep): every
    # element of O, LSE, dQ, dK and dV against the oracle.
    w = _wl(1, 1, 16384, 16384, 128, seed=77 + int(causal), causal=causal)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    dq, dk, dv = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_whole(x, o, lse, w.scale, causal)
    _check_bwd(x, o, dq, dk, dv, w.scale, causal)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_fwd_bwd_whole(d, causal):
    # 8 x 64 = 512 heads of 80 queries against 72 keys: thousands of small,
    # ragged tiles (head decoding and the XCD remap across a large grid; with
    # the mask the first 8 queries of every head see no key).
    w = _wl(8, 64, 80, 72, d, seed=300 + d + int(causal), causal=causal)
    x = _cuda(make_inputs(w, with_grad_output=True))
    o, lse = ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=causal)
    dq, dk, dv = ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=causal)
    torch.cuda.synchronize()
    _check_whole(x, o, lse, w.scale, causal)
    q, k, v, do = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    ref = backward_all(q, k, v, to_f64(o), do, w.scale, causal=causal)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        got = to_f64(got)
        for (b, h) in np.ndindex(w.B, w.H):
            _assert_grad(f"{name}[{b},{h}]", got[b, h], want[b, h])
    if causal:
        assert torch.all(dq[:, :, :8] == 0)
