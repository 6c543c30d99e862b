"""Host logic of bench.py and of the build, checked without a GPU.

bench.py's CPU leg is the only place the benchmark runs the oracle: it times
the oracle on whole heads and checks every measured output against it. Here
it is fed outputs that are the oracle's own result rounded to bf16 (within
the bars, so the check must pass) and the same with one element moved by
0.1 (outside the 2e-2 bar, so it must fail). The debug build of the library
(every LDS transfer ordered by the compiler) must export what the release
build exports.
"""

import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench  # noqa: E402
import tiled_attention_17_amd as ta  # noqa: E402
from oracle import attention_backward, attention_forward  # noqa: E402
from tiled_attention_17_amd.workloads import Workload, make_inputs, to_f64  # noqa: E402


def _fwd_outputs(w, x, causal=False):
    ro, rl = attention_forward(*(to_f64(x[n]) for n in ("q", "k", "v")), w.scale, causal=causal)
    return torch.from_numpy(ro).to(torch.bfloat16), torch.from_numpy(rl).to(torch.float32)


def _legs(perturb):
    w = Workload("mha_bf16_b1h2_n64_d64", 1, 2, 64, 64, "bf16", seed=3)
    x = make_inputs(w)
    o, lse = _fwd_outputs(w, x)
    wb = Workload("fwdbwd_bf16_b1h2_n64_d64", 1, 2, 64, 64, "bf16", seed=5, backward=True)
    xb = make_inputs(wb)
    ob, lb = _fwd_outputs(wb, xb)
    grads = [torch.from_numpy(g).to(torch.bfloat16)
             for g in attention_backward(*(to_f64(xb[n]) for n in ("q", "k", "v", "do")), wb.scale)]
    if perturb:
        grads[1][0, 1, 5, 7] += 0.1
    checks = [{"name": wb.name, "kind": "bwd", "x": xb, "scale": wb.scale, "heads": [(0, 0), (0, 1)],
               "o": ob, "lse": lb, "grads": grads}]
    return bench.cpu_leg(w, x, o, lse, 0.05, checks)


def test_cpu_leg_passes_oracle_outputs():
    baseline, ver = _legs(perturb=False)
    assert ver["pass"], ver
    assert baseline["kind"] == "oracle" and baseline["value"] > 0 and baseline["cores"] >= 1
    assert baseline["cpu_model"] and baseline["blas"]
    r = ver["workloads"]["mha_bf16_b1h2_n64_d64"]
    assert r["heads_checked"] == 2 and r["max_abs_err_O"] <= 2e-2 and r["max_abs_err_LSE"] <= 1e-3


def test_cpu_leg_fails_a_planted_gradient_error():
    _, ver = _legs(perturb=True)
    assert not ver["pass"]
    r = ver["workloads"]["fwdbwd_bf16_b1h2_n64_d64"]
    assert not r["pass"] and r["max_abs_err_dK"] > 0.09


@pytest.mark.skipif(not os.path.exists(os.path.join(os.path.dirname(ta.LIB_PATH), "libtiledattn_ordered.so")),
                    reason="debug library not built")
def test_ordered_debug_library_exports_the_same_entry_points():
    rel = ctypes.CDLL(os.path.join(os.path.dirname(ta.LIB_PATH), "libtiledattn.so"))
    dbg = ctypes.CDLL(os.path.join(os.path.dirname(ta.LIB_PATH), "libtiledattn_ordered.so"))
    for name in ("attn_fwd", "attn_fwd_ex", "attn_merge", "attn_bwd", "attn_bwd_ex", "attn_bwd_ex_noalloc",
                 "attn_fwd_mxfp8", "attn_quantize_mxfp8", "attn_matmul_nt", "attn_version"):
        assert hasattr(rel, name) and hasattr(dbg, name), name
    assert rel.attn_version() == dbg.attn_version()
