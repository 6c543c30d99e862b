#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step = one forward pass (attn_fwd through the C ABI) over the headline
workload: B=2, H=16, N=4096, d=128, bf16 Q, K, V ~ N(0,1), scale 1/sqrt(d),
inputs resident in device memory before the timed region. Prints one JSON
line with whole-job throughput (TFLOP/s at 4*B*H*N^2*d FLOPs per step), the
roofline position of the kernel (timed live with HIP events on its launch
stream), and the float64 CPU oracle timed on a bounded sample of the same
workload on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) + % of MI355X bf16 MFMA peak, N=4096 d=128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "tiled_attention_17_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "tile_common.h", "device_common.h")]


def kernel_source_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter run, if it was taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_digest():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, x, seconds):
    """The float64 oracle on whole heads of the workload until ~`seconds` elapse."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_forward
    from tiled_attention_17_amd.perfmodel import attn_fwd_flops
    from tiled_attention_17_amd.workloads import to_f64

    q, k, v = (to_f64(x[n]) for n in ("q", "k", "v"))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    # whole heads, cycling over the workload's heads until the budget is spent
    done, t0 = 0, time.perf_counter()
    while True:
        b, h = heads[done % len(heads)]
        attention_forward(q[b, h], k[b, h], v[b, h], w.scale)
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    flops = attn_fwd_flops(1, done, w.N, w.d)
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} head evaluations (the workload has {len(heads)} heads) of {w.name} "
                  f"(float64 NumPy, S and P materialised), "
                  f"{el:.1f} s; BLAS threads {threads}, host CPUs {len(os.sched_getaffinity(0))}",
        "seconds": el,
    }


def _time_ms(fn, stream, warm, n):
    """Average milliseconds of fn() over n calls after warm calls (HIP events on `stream`)."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def measure_ex(ta, pm, dev, stream, n):
    """Figures of the masked and unequal-length paths (not the headline metric).

    causal: forward and backward at the headline shape, TFLOP/s over the
    visible (query, key) pairs (4 d resp. 10 d FLOPs per pair); shard: one
    device's 2048 queries of a 16384-long sequence against all its keys
    (library-chosen key splits); decode: one query per sequence against 8192
    keys, bound by reading K and V (GB/s against 8 TB/s); mxfp8: the MXFP8
    forward at the headline shape against the fp8 dense peak.
    """
    import torch

    from tiled_attention_17_amd.workloads import EXTRA_WORKLOADS, make_inputs

    out = {}
    peak = pm.MI355X_PEAK_FLOPS["bf16"] / 1e12
    for w in EXTRA_WORKLOADS:
        x = {k: t.to(dev) for k, t in make_inputs(w, with_grad_output=w.causal).items()}
        o = torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        splits = 1 if w.causal else ta.attn_fwd_ex_auto_splits(w.B, w.H, w.Nq, w.Nk, w.d)
        need = ta.attn_fwd_ex_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def fwd():
            ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=w.causal, num_splits=splits,
                           out=o, lse=lse, workspace=ws)

        ms = _time_ms(fwd, stream, 3 * n, n)
        fl = pm.attn_fwd_flops_masked(w.B, w.H, w.Nq, w.Nk, w.d, w.causal)
        nbytes = pm.attn_fwd_bytes_ex(w.B, w.H, w.Nq, w.Nk, w.d, 2)
        r = {"workload": w.name, "splits": splits, "ms": ms, "tflops": fl / (ms * 1e-3) / 1e12,
             "pct_of_bf16_dense_peak": 100.0 * fl / (ms * 1e-3) / 1e12 / peak,
             "gb_per_s": nbytes / (ms * 1e-3) / 1e9,
             "pct_of_hbm": 100.0 * nbytes / (ms * 1e-3) / pm.MI355X_HBM_BYTES_PER_S}
        if w.causal:
            g = [torch.empty_like(x["q"]) for _ in range(3)]
            bws = torch.empty(ta.attn_bwd_workspace_bytes(w.B, w.H, w.Nq, w.d), dtype=torch.uint8,
                              device=dev)

            def bwd():
                ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=True,
                               dq=g[0], dk=g[1], dv=g[2], workspace=bws)

            bms = _time_ms(bwd, stream, 3, max(3, n // 5))
            bfl = pm.attn_bwd_flops_masked(w.B, w.H, w.Nq, w.Nk, w.d, True)
            r.update({"bwd_ms": bms, "bwd_tflops": bfl / (bms * 1e-3) / 1e12})
            del g, bws
        out[w.name.split("_")[0]] = r
        del x, o, lse, ws

    # MXFP8 forward at the headline shape: inputs quantized beforehand and
    # resident as MXFP8 (the quantizer's own time reported separately)
    from tiled_attention_17_amd.workloads import HEADLINE
    w = HEADLINE
    x = {k: t.to(dev) for k, t in make_inputs(w).items()}
    q8, qs = ta.attn_quantize_mxfp8(x["q"])
    k8, ks = ta.attn_quantize_mxfp8(x["k"])
    vt8, vts = ta.attn_quantize_mxfp8(x["v"], transpose=True)
    o = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    ms = _time_ms(lambda: ta.attn_fwd_mxfp8(q8, qs, k8, ks, vt8, vts, w.scale, out=o, lse=lse), stream,
                  3 * n, n)
    qms = _time_ms(lambda: (ta.attn_quantize_mxfp8(x["q"]), ta.attn_quantize_mxfp8(x["k"]),
                            ta.attn_quantize_mxfp8(x["v"], transpose=True)), stream, 3, n)
    fl = pm.attn_fwd_flops(w.B, w.H, w.N, w.d)
    out["mxfp8"] = {"workload": w.name + " (MXFP8 Q, K, V^T)", "ms": ms, "tflops": fl / (ms * 1e-3) / 1e12,
                    "pct_of_fp8_dense_peak": 100.0 * fl / (ms * 1e-3) / pm.MI355X_PEAK_FLOPS["fp8"],
                    "quantize_q_k_vt_ms": qms}
    return out


def measure_configs(ta, pm, dev, stream, n):
    """The other forward configurations (not the headline metric).

    fp32 single head (B=1 H=1 N=256 d=64, against the fp32 MFMA peak), the
    d = 64 multi-head case (B=4 H=8 N=1024) and the long sequence with
    spread scores (B=1 H=16 N=16384 d=128, Q ~ N(0, 3^2)), each with
    library-chosen tiles and one launch per step.
    """
    import torch

    from tiled_attention_17_amd.workloads import WORKLOADS, make_inputs

    out = {}
    for w, key in ((WORKLOADS[0], "fp32_small"), (WORKLOADS[1], "d64"), (WORKLOADS[3], "long")):
        x = {k: t.to(dev) for k, t in make_inputs(w).items()}
        o = torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
        reps = n if w.N <= 4096 else max(5, n // 10)
        ms = _time_ms(lambda: ta.attn_fwd(x["q"], x["k"], x["v"], w.scale, out=o, lse=lse), stream,
                      3 * reps, reps)
        fl = pm.attn_fwd_flops(w.B, w.H, w.N, w.d)
        dt = "fp32" if w.dtype == "fp32" else "bf16"
        peak = pm.MI355X_PEAK_FLOPS[dt] / 1e12
        tf = fl / (ms * 1e-3) / 1e12
        out[key] = {"workload": w.name, "ms": ms, "tflops": tf, f"pct_of_{dt}_dense_peak": 100.0 * tf / peak}
        del x, o, lse
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The warm-up is long on purpose: under sustained load the MI355X raises
    # its shader clock over tens of milliseconds (measured on this kernel:
    # ~1.85 GHz after 10 launches, a steady ~2.05 GHz after ~100 ms), so a
    # short warm-up times the clock ramp rather than the kernel.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU work budget of the oracle baseline (0 disables it)")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward figures in 'extra'")
    ap.add_argument("--no-ex", action="store_true",
                    help="skip the causal / unequal-length / decoding / other-configuration figures in 'extra'")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the attention path has no multi-GPU code.", file=sys.stderr)
        sys.exit(2)

    import torch

    import tiled_attention_17_amd as ta
    from tiled_attention_17_amd import perfmodel as pm
    from tiled_attention_17_amd.workloads import HEADLINE, WORKLOADS, make_inputs

    w = HEADLINE
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_cpu = make_inputs(w)
    x = {n: t.to(dev) for n, t in x_cpu.items()}
    o = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        ta.attn_fwd(x["q"], x["k"], x["v"], w.scale, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(K):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_launch = [ev[i].elapsed_time(ev[i + 1]) for i in range(K)]
    total_ms = ev[0].elapsed_time(ev[K])
    ms_per_step = total_ms / K
    flops = pm.attn_fwd_flops(w.B, w.H, w.N, w.d)
    value = flops / (ms_per_step * 1e-3) / 1e12
    kernel_ms = sum(per_launch) / K
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = pm.MI355X_PEAK_FLOPS["bf16"] / 1e12

    extra = {
        "pct_of_bf16_dense_peak": 100.0 * value / peak,
        "kernel_ms_min": min(per_launch),
        "kernel_ms_median": sorted(per_launch)[K // 2],
        "algorithmic_bytes_per_launch": pm.attn_fwd_bytes(w.B, w.H, w.N, w.d, 2),
    }
    if not args.no_bwd:
        wb = WORKLOADS[4]
        xb = {n: t.to(dev) for n, t in make_inputs(wb).items()}
        ob, lb = ta.attn_fwd(xb["q"], xb["k"], xb["v"], wb.scale)
        g = [torch.empty_like(ob) for _ in range(3)]
        ws = torch.empty(ta.attn_bwd_workspace_bytes(wb.B, wb.H, wb.N, wb.d), dtype=torch.uint8,
                         device=dev)

        def bstep():
            ta.attn_bwd(xb["q"], xb["k"], xb["v"], ob, xb["do"], lb, wb.scale, dq=g[0], dk=g[1],
                        dv=g[2], workspace=ws)

        for _ in range(3):
            bstep()
        torch.cuda.synchronize()
        nb = max(3, K // 5)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(nb):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / nb
        extra.update({
            "bwd_workload": wb.name,
            "bwd_ms": bms,
            "bwd_tflops_10BHN2d": pm.attn_bwd_flops(wb.B, wb.H, wb.N, wb.d) / (bms * 1e-3) / 1e12,
            "fwd_plus_bwd_tflops_14BHN2d": pm.attn_fwd_flops(wb.B, wb.H, wb.N, wb.d) * 3.5
            / ((ms_per_step + bms) * 1e-3) / 1e12,
        })
        del xb, ob, lb, g, ws

    if not args.no_ex:
        extra.update(measure_ex(ta, pm, dev, stream, max(20, K // 4)))
        extra.update(measure_configs(ta, pm, dev, stream, max(20, K // 4)))

    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "scale": w.scale, "inputs": "Q,K,V iid N(0,1), seed 3, bf16 RNE",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic},
        "cpu_baseline": None,
        "extra": extra,
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(w, x_cpu, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
