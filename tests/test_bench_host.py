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
import json
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
    for name in ("attn_fwd", "attn_fwd_ex", "attn_fwd_ex_timed", "attn_merge", "attn_bwd", "attn_bwd_ex", "attn_bwd_ex_noalloc",
                 "attn_fwd_mxfp8", "attn_quantize_mxfp8", "attn_matmul_nt", "attn_version"):
        assert hasattr(rel, name) and hasattr(dbg, name), name
    assert rel.attn_version() == dbg.attn_version()


def test_trace_summary_picks_the_timed_launches(tmp_path):
    # A synthetic kernel trace in bench.py's launch order: settle + warm-up
    # launches of the headline forward, the timed region's back-to-back
    # launches (300 us), the launches with kernel-bound events (250 us), then
    # other kernels and later forward launches of other shapes.
    from tiled_attention_17_amd import profiling
    settle, warm, steps = 7, 2, 4
    fwd = "void tattn::attn_fwd_bf16_pingpong_kernel<128, 128>(tattn::FwdParams)"
    durs = [400_000] * (settle + warm) + [300_000] * steps + [250_000, 240_000, 260_000, 250_000]
    rows, t = [], 0
    for i, ns in enumerate(durs):
        rows.append((i + 1, fwd, t, t + ns))
        t += ns + 1000
    rows += [(len(rows) + 1, "void tattn::attn_bwd_dkdv_kernel<128>(tattn::BwdParams)", t, t + 90_000),
             (len(rows) + 2, fwd, t + 100_000, t + 900_000)]
    trace = tmp_path / "run"
    trace.mkdir()
    with open(trace / "bench_kernel_trace.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for r in rows:
            f.write(f'{r[0]},"{r[1]}",{r[2]},{r[3]}\n')
    flops = 4 * 2 * 16 * 4096 ** 2 * 128
    line = {"value": 1.0, "ms_per_step": 0.301, "steps": steps, "warmup": warm,
            "config": {"workload": "w", "B": 2, "H": 16, "N": 4096, "d": 128},
            "roofline": {"peak": 2500.0, "achieved": flops / 251e-6 / 1e12, "frac": flops / 251e-6 / 2.5e15},
            "extra": {"settle_launches": settle, "settle_ms": 3.0, "kernel_ms_mean": 0.251,
                      "kernel_ms_median": 0.251, "kernel_ms_min": 0.241, "interval_ms_mean": 0.301}}
    line_file = tmp_path / "line.txt"
    line_file.write_text("log text\n" + json.dumps(line) + "\n")
    out = tmp_path / "summary.md"
    profiling.summarize_bench(str(trace), str(line_file), "python3 bench.py", str(out))
    text = out.read_text()
    assert "| timed region: average duration / time per launch | 300.0 us |" in text
    assert "| kernel-bound events: average duration | 250.0 us | 251.0 us |" in text
    assert "| min duration | 240.0 us | 241.0 us |" in text
    assert f"{flops / 250e-6 / 2.5e15:.4f}" in text
    assert "launches 14..17" in text
