#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step = one forward pass (attn_fwd through the C ABI) over the headline
workload: B=2, H=16, N=4096, d=128, bf16 Q, K, V ~ N(0,1), scale 1/sqrt(d),
inputs resident in device memory before the timed region. Prints one JSON
line with whole-job throughput (TFLOP/s at 4*B*H*N^2*d FLOPs per step), the
roofline position of the kernel (timed live with HIP events on its launch
stream), the float64 CPU oracle timed on a bounded sample of the same
workload on this host's cores, and, in "extra", the other workloads' figures
and the check of every measured output against the oracle.

Timing recipe (Lecture 17 page, §10.1-§10.2: warm up, time with events on the
launch stream, repeat, verify the outputs):
  * clock settle: under sustained load the MI355X raises its shader clock
    over tens of milliseconds, so before the timed region each measurement
    launches its kernel until --settle-ms of GPU time have passed (whatever
    --warmup says), then --warmup more launches;
  * every timed launch has its own start and end events, so the per-launch
    kernel time (mean, median, min) is reported beside the whole-region step
    time; for the forward launches of the headline and of the fp32, d = 64
    and long-sequence workloads the library binds the two events to the
    start and end of the attention kernel's dispatch (attn_fwd_ex_timed), so
    they time the kernel alone and put no event commands between the
    launches; the other measurements record their events around the call;
  * the short configurations (fp32 single head, d = 64) are also timed cold
    (a 1 GiB scratch write between launches evicts the L2s and the Infinity
    Cache, and each launch is timed on its own) and back to back (a burst of
    launches between one pair of events, without the per-launch events whose
    own overhead is a sizeable part of a launch of a few microseconds);
  * the outputs of the timed launches are kept and compared with the oracle
    in the CPU leg (whole heads of the headline workload, every head of the
    d = 64 and fp32 workloads, sampled rows of the long sequence, sampled
    heads of the backward).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms T]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·d) + % of MI355X bf16 MFMA peak, N=4096 d=128"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "tiled_attention_17_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "tile_common.h", "device_common.h")]
COLD_SCRATCH_BYTES = 1 << 30


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


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def time_launches(fn, stream, n, warm, settle_ms, timed_fn=None):
    """Launch fn until settle_ms of GPU time pass, then warm more, then time n launches.

    Without timed_fn each timed launch is bracketed by its own start and end
    events on `stream`. Returns per-launch mean / median / min
    (kernel_ms_*), the whole region's time per launch (ms_per_launch) and
    what the settle did.

    With timed_fn (fn's call made through attn_fwd_ex_timed, given a start and
    a stop event that the library binds to its attention kernel's dispatch):
      * the timed region holds the n launches back to back with only their
        stop events bound, which adds no command between them (a bound start
        event is a marker command of its own, ≈5 µs per launch):
        ms_per_launch is the rate of an uninterrupted stream of launches, and
        interval_ms_* the time from one kernel's end to the next one's
        (its duration plus the dispatch gap before it);
      * then n more launches with both events bound give each kernel's own
        duration (kernel_ms_*), what a kernel trace shows.
    """
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    torch.cuda.synchronize()
    spent, settle_launches, batch = 0.0, 0, 2
    while spent < settle_ms:
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(batch):
            fn()
        b.record(stream)
        b.synchronize()
        ms = a.elapsed_time(b)
        spent += ms
        settle_launches += batch
        if ms < 20.0:  # keep the queue full without syncing after every few launches
            batch = min(2 * batch, 4096)
    for _ in range(warm):
        fn()
    starts, ends = [ev() for _ in range(n)], [ev() for _ in range(n)]
    t0, t1 = ev(), ev()
    r = {"launches": n, "warmup": warm, "settle_ms": spent, "settle_launches": settle_launches}
    if timed_fn is None:
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(n):
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
        t1.record(stream)
        torch.cuda.synchronize()
    else:
        stops = [ev() for _ in range(n)]
        for e in starts + ends + stops:  # torch creates an event's HIP handle on its first record
            e.record(stream)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(n):
            timed_fn(None, stops[i])
        t1.record(stream)
        for i in range(n):
            timed_fn(starts[i], ends[i])
        torch.cuda.synchronize()
        iv = sorted(stops[i - 1].elapsed_time(stops[i]) for i in range(1, n))
        if iv:
            r.update(interval_ms_mean=sum(iv) / len(iv), interval_ms_median=iv[len(iv) // 2],
                     interval_ms_min=iv[0])
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    r.update(kernel_ms_mean=sum(per) / n, kernel_ms_median=per[n // 2], kernel_ms_min=per[0],
             ms_per_launch=t0.elapsed_time(t1) / n)
    return r


def time_burst(fn, stream, n):
    """Time per launch of n back-to-back launches between one pair of events.

    For kernels of a few microseconds the per-launch events of time_launches
    add their own overhead to each launch; a burst without them shows what a
    stream of such launches costs (the dispatch gaps between them included).
    """
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    b.synchronize()
    return {"ms_per_launch": a.elapsed_time(b) / n, "launches": n}


def time_cold(fn, stream, n, scratch):
    """Per-launch time with the caches evicted before each launch (1 GiB scratch write)."""
    import torch
    per = []
    for i in range(n):
        scratch.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        b.synchronize()
        per.append(a.elapsed_time(b))
    per.sort()
    return {"kernel_ms_median": per[n // 2], "kernel_ms_mean": sum(per) / n, "kernel_ms_min": per[0],
            "launches": n, "evict_bytes": scratch.numel()}


def _rates(pm, flops, nbytes, ms, dt):
    peak = pm.MI355X_PEAK_FLOPS[dt]
    return {"tflops": flops / (ms * 1e-3) / 1e12, f"pct_of_{dt}_dense_peak": 100.0 * flops / (ms * 1e-3) / peak,
            "gb_per_s": nbytes / (ms * 1e-3) / 1e9,
            "pct_of_hbm": 100.0 * nbytes / (ms * 1e-3) / pm.MI355X_HBM_BYTES_PER_S}


# ---------------------------------------------------------------------------
# measurements (each returns its figures and what the CPU leg should check)
# ---------------------------------------------------------------------------

def _rows_sample(n, count, seed):
    import numpy as np
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, n // 2, n - 1], rng.integers(0, n, count)]))


def measure_backward(ta, pm, dev, stream, n, settle_ms, checks):
    import torch

    from tiled_attention_17_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[4]
    x_cpu = make_inputs(w)
    x = {k: t.to(dev) for k, t in x_cpu.items()}
    o, lse = ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
    g = [torch.empty_like(o) for _ in range(3)]
    ws = torch.empty(max(ta.attn_bwd_workspace_bytes(w.B, w.H, w.N, w.d), 16), dtype=torch.uint8, device=dev)

    def bwd():
        ta.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, dq=g[0], dk=g[1], dv=g[2], workspace=ws)

    t = time_launches(bwd, stream, n, 3, settle_ms)
    ms = t["kernel_ms_mean"]
    fl = pm.attn_bwd_flops(w.B, w.H, w.N, w.d)
    nb = pm.attn_bwd_bytes(w.B, w.H, w.N, w.d, 2)
    r = {"workload": w.name, **t, **_rates(pm, fl, nb, ms, "bf16"),
         "flops_counted": "10·B·H·N²·d"}
    # The same calls back to back without events between them (each call is
    # two launches; per-call events add their own commands to every call).
    bb = time_burst(bwd, stream, n)
    r["back_to_back"] = {**bb, **_rates(pm, fl, nb, bb["ms_per_launch"], "bf16")}
    # The forward of the same inputs, for the forward + backward total at
    # 14·B·H·N²·d (the forward's kernel time with kernel-bound events).
    fo, flse = torch.empty_like(o), torch.empty_like(lse)

    def fwd():
        ta.attn_fwd(x["q"], x["k"], x["v"], w.scale, out=fo, lse=flse)

    def fwd_timed(start, stop):
        ta.attn_fwd_ex_timed(x["q"], x["k"], x["v"], start, stop, w.scale, out=fo, lse=flse)

    tf = time_launches(fwd, stream, n, 3, 0.0, fwd_timed)
    fwd_ms = tf["kernel_ms_mean"]
    r["fwd_kernel_ms_mean"] = fwd_ms
    r["fwd_bwd_ms"] = fwd_ms + ms
    r["fwd_bwd_tflops"] = (pm.attn_fwd_flops(w.B, w.H, w.N, w.d) + fl) / ((fwd_ms + ms) * 1e-3) / 1e12
    r["fwd_bwd_flops_counted"] = "14·B·H·N²·d"
    del fo, flse
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    checks.append({"name": w.name, "kind": "bwd", "x": x_cpu, "scale": w.scale, "heads": heads,
                   "o": o.cpu(), "lse": lse.cpu(), "grads": [t.cpu() for t in g]})
    return r


def measure_configs(ta, pm, dev, stream, n, settle_ms, checks):
    """fp32 single head (cfg 1), d = 64 multi-head (cfg 2), long sequence with spread scores (cfg 4)."""
    import torch

    from tiled_attention_17_amd.workloads import WORKLOADS, make_inputs
    out = {}
    scratch = torch.empty(COLD_SCRATCH_BYTES, dtype=torch.uint8, device=dev)
    for w, key in ((WORKLOADS[0], "fp32_small"), (WORKLOADS[1], "d64"), (WORKLOADS[3], "long")):
        x_cpu = make_inputs(w)
        x = {k: t.to(dev) for k, t in x_cpu.items()}
        o = torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def fwd():
            ta.attn_fwd(x["q"], x["k"], x["v"], w.scale, out=o, lse=lse)

        def fwd_timed(start, stop):
            ta.attn_fwd_ex_timed(x["q"], x["k"], x["v"], start, stop, w.scale, out=o, lse=lse)

        long = w.N > 4096
        t = time_launches(fwd, stream, max(5, n // 10) if long else n, 3, settle_ms, fwd_timed)
        dt = "fp32" if w.dtype == "fp32" else "bf16"
        eb = 4 if dt == "fp32" else 2
        fl = pm.attn_fwd_flops(w.B, w.H, w.N, w.d)
        nb = pm.attn_fwd_bytes(w.B, w.H, w.N, w.d, eb)
        r = {"workload": w.name, "cache": "warm (inputs resident in L2 / Infinity Cache across launches)",
             **t, **_rates(pm, fl, nb, t["kernel_ms_mean"], dt), "algorithmic_bytes": nb}
        if not long:
            bb = time_burst(fwd, stream, 10 * n)
            r["back_to_back"] = {**bb, **_rates(pm, fl, nb, bb["ms_per_launch"], dt)}
            c = time_cold(fwd, stream, n, scratch)
            r["cold"] = {**c, **_rates(pm, fl, nb, c["kernel_ms_median"], dt)}
        out[key] = r
        chk = {"name": w.name, "kind": "fwd", "x": x_cpu, "scale": w.scale}
        if long:  # sampled rows of every head; whole-output parity is in the tests
            rows = _rows_sample(w.N, 60, 4)
            chk.update(rows=rows, o=o[:, :, rows].cpu(), lse=lse[:, :, rows].cpu())
        else:
            chk.update(o=o.cpu(), lse=lse.cpu())
        checks.append(chk)
        del x, o, lse
    del scratch
    return out


def measure_ex(ta, pm, dev, stream, n, settle_ms, checks):
    """Causal, query shard, decode (masked and unequal-length paths) and the MXFP8 forward."""
    import torch

    from tiled_attention_17_amd.workloads import EXTRA_WORKLOADS, HEADLINE, make_inputs
    out = {}
    for w in EXTRA_WORKLOADS:
        x_cpu = make_inputs(w, with_grad_output=w.causal)
        x = {k: t.to(dev) for k, t in x_cpu.items()}
        o = torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        splits = 1 if w.causal else ta.attn_fwd_ex_auto_splits(w.B, w.H, w.Nq, w.Nk, w.d)
        need = ta.attn_fwd_ex_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d, splits)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

        def fwd():
            ta.attn_fwd_ex(x["q"], x["k"], x["v"], w.scale, causal=w.causal, num_splits=splits,
                           out=o, lse=lse, workspace=ws)

        t = time_launches(fwd, stream, n, 3, settle_ms)
        fl = pm.attn_fwd_flops_masked(w.B, w.H, w.Nq, w.Nk, w.d, w.causal)
        nb = pm.attn_fwd_bytes_ex(w.B, w.H, w.Nq, w.Nk, w.d, 2)
        r = {"workload": w.name, "splits": splits, **t, **_rates(pm, fl, nb, t["kernel_ms_mean"], "bf16")}
        if w.causal:
            g = [torch.empty_like(x["q"]) for _ in range(3)]
            bws = torch.empty(max(ta.attn_bwd_workspace_bytes(w.B, w.H, w.Nq, w.d), 16), dtype=torch.uint8,
                              device=dev)

            def bwd():
                ta.attn_bwd_ex(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale, causal=True,
                               dq=g[0], dk=g[1], dv=g[2], workspace=bws)

            tb = time_launches(bwd, stream, n, 3, settle_ms)
            bfl = pm.attn_bwd_flops_masked(w.B, w.H, w.Nq, w.Nk, w.d, True)
            r["bwd"] = {**tb, "tflops": bfl / (tb["kernel_ms_mean"] * 1e-3) / 1e12,
                        "pct_of_bf16_dense_peak": 100.0 * bfl / (tb["kernel_ms_mean"] * 1e-3)
                        / pm.MI355X_PEAK_FLOPS["bf16"]}
            del g, bws
        out[w.name.split("_")[0]] = r
        heads = [(0, 0), (w.B - 1, w.H - 1)]
        checks.append({"name": w.name, "kind": "fwd", "x": x_cpu, "scale": w.scale, "causal": w.causal,
                       "heads": heads, "o": o.cpu(), "lse": lse.cpu()})
        del x, o, lse, ws

    # MXFP8 forward at the headline shape: inputs quantized beforehand and
    # resident as MXFP8 (the quantizer's own time reported separately)
    w = HEADLINE
    x = {k: t.to(dev) for k, t in make_inputs(w).items()}
    q8, qs = ta.attn_quantize_mxfp8(x["q"])
    k8, ks = ta.attn_quantize_mxfp8(x["k"])
    vt8, vts = ta.attn_quantize_mxfp8(x["v"], transpose=True)
    o = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    t = time_launches(lambda: ta.attn_fwd_mxfp8(q8, qs, k8, ks, vt8, vts, w.scale, out=o, lse=lse), stream,
                      n, 3, settle_ms)
    tq = time_launches(lambda: (ta.attn_quantize_mxfp8(x["q"]), ta.attn_quantize_mxfp8(x["k"]),
                                ta.attn_quantize_mxfp8(x["v"], transpose=True)), stream, n, 3, 0.0)
    fl = pm.attn_fwd_flops(w.B, w.H, w.N, w.d)
    out["mxfp8"] = {"workload": w.name + " (MXFP8 Q, K, V^T)", **t,
                    "tflops": fl / (t["kernel_ms_mean"] * 1e-3) / 1e12,
                    "pct_of_fp8_dense_peak": 100.0 * fl / (t["kernel_ms_mean"] * 1e-3) / pm.MI355X_PEAK_FLOPS["fp8"],
                    "quantize_q_k_vt_ms": tq["ms_per_launch"]}
    return out


# ---------------------------------------------------------------------------
# CPU leg: the oracle as a timed baseline, and the check of the measured outputs
# ---------------------------------------------------------------------------

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _max_abs(a, b):
    import numpy as np
    return float(np.max(np.abs(a - b))) if b.size else 0.0


def _lse_err(got, want):
    import numpy as np
    empty = np.isneginf(want)
    if not np.array_equal(np.isneginf(got), empty):
        return float("inf")
    return _max_abs(got[~empty], want[~empty]) if (~empty).any() else 0.0


def cpu_leg(w, x_cpu, o_gpu, lse_gpu, seconds, checks):
    """(cpu_baseline, verification) -- the only part of bench.py that runs the oracle.

    Baseline: the float64 oracle on whole heads of the headline workload,
    cycling over its heads until ~`seconds` of oracle time are spent; each
    head it computes is also compared with the GPU's output of the timed
    launches. Verification: every record in `checks` against the oracle.
    Bars: bf16 O, dQ, dK, dV max abs error <= 2e-2, fp32 O <= 1e-5, LSE <= 1e-3.
    """
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_backward, attention_forward
    from tiled_attention_17_amd.perfmodel import attn_fwd_flops
    from tiled_attention_17_amd.workloads import to_f64

    q, k, v = (to_f64(x_cpu[n]) for n in ("q", "k", "v"))
    go, gl = to_f64(o_gpu), to_f64(lse_gpu)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, el, errs = 0, 0.0, {}
    while el < seconds:
        b, h = heads[done % len(heads)]
        t0 = time.perf_counter()
        ro, rl = attention_forward(q[b, h], k[b, h], v[b, h], w.scale)
        el += time.perf_counter() - t0
        done += 1
        if (b, h) not in errs:
            errs[(b, h)] = (_max_abs(go[b, h], ro), _max_abs(gl[b, h], rl))
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    vendor = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas) or "unknown"
    flops = attn_fwd_flops(1, done, w.N, w.d)
    baseline = {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} head evaluations (the workload has {len(heads)} heads) of {w.name} "
                  f"(float64 NumPy, S and P materialised), {el:.1f} s of oracle time; BLAS threads {threads}, "
                  f"host CPUs {len(os.sched_getaffinity(0))}",
        "seconds": el,
        "cpu_model": _cpu_model(),
        "blas": vendor,
    }

    bars = {"bf16": 2e-2, "fp32": 1e-5, "lse": 1e-3}
    ver = {w.name: {"heads_checked": len(errs), "rows": "all",
                    "max_abs_err_O": max(e[0] for e in errs.values()),
                    "max_abs_err_LSE": max(e[1] for e in errs.values())}}
    for c in checks:
        t0 = time.perf_counter()
        x = {n: to_f64(t) for n, t in c["x"].items()}
        o, lse = to_f64(c["o"]), to_f64(c["lse"])
        B, H = x["q"].shape[:2]
        hs = c.get("heads") or [(b, h) for b in range(B) for h in range(H)]
        rows = c.get("rows")
        eo = el_ = 0.0
        grads = [0.0, 0.0, 0.0]
        for (b, h) in hs:
            qi = x["q"][b, h] if rows is None else x["q"][b, h][rows]
            ro, rl = attention_forward(qi, x["k"][b, h], x["v"][b, h], c["scale"], causal=c.get("causal", False))
            eo = max(eo, _max_abs(o[b, h], ro))
            el_ = max(el_, _lse_err(lse[b, h], rl))
            if c["kind"] == "bwd":
                ref = attention_backward(x["q"][b, h], x["k"][b, h], x["v"][b, h], x["do"][b, h], c["scale"])
                for i, (gt, rt) in enumerate(zip(c["grads"], ref)):
                    grads[i] = max(grads[i], _max_abs(to_f64(gt[b, h]), rt))
        r = {"heads_checked": len(hs), "rows": "all" if rows is None else f"{len(rows)} sampled per head",
             "max_abs_err_O": eo, "max_abs_err_LSE": el_, "oracle_s": time.perf_counter() - t0}
        if c["kind"] == "bwd":
            r.update({"max_abs_err_dQ": grads[0], "max_abs_err_dK": grads[1], "max_abs_err_dV": grads[2]})
        ver[c["name"]] = r
    ok = True
    for name, r in ver.items():
        tol = bars["fp32"] if "fp32" in name else bars["bf16"]
        good = all(r.get(f"max_abs_err_{n}", 0.0) <= tol for n in ("O", "dQ", "dK", "dV")) \
            and r["max_abs_err_LSE"] <= bars["lse"]
        r["pass"] = bool(good)
        ok = ok and good
    return baseline, {"bars": bars, "pass": ok, "workloads": ver}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="GPU time of headline launches before the warm-up (clock settle)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle time of the CPU baseline (0 disables the CPU leg and the output check)")
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
    from tiled_attention_17_amd.workloads import HEADLINE, make_inputs

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

    def step_timed(start, stop):
        ta.attn_fwd_ex_timed(x["q"], x["k"], x["v"], start, stop, w.scale, out=o, lse=lse)

    K = args.steps
    t = time_launches(step, stream, K, args.warmup, args.settle_ms, step_timed)
    o_timed, lse_timed = o.cpu(), lse.cpu()  # every launch writes the same result
    ms_per_step = t["ms_per_launch"]
    flops = pm.attn_fwd_flops(w.B, w.H, w.N, w.d)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (t["kernel_ms_mean"] * 1e-3) / 1e12
    peak = pm.MI355X_PEAK_FLOPS["bf16"] / 1e12
    nbytes = pm.attn_fwd_bytes(w.B, w.H, w.N, w.d, 2)

    extra = {
        "pct_of_bf16_dense_peak": 100.0 * value / peak,
        "settle_ms": t["settle_ms"],
        "settle_launches": t["settle_launches"],
        "kernel_ms_mean": t["kernel_ms_mean"],
        "kernel_ms_median": t["kernel_ms_median"],
        "kernel_ms_min": t["kernel_ms_min"],
        "interval_ms_mean": t.get("interval_ms_mean"),
        "interval_ms_median": t.get("interval_ms_median"),
        "algorithmic_bytes_per_launch": nbytes,
        "gb_per_s": nbytes / (t["kernel_ms_mean"] * 1e-3) / 1e9,
        "timing": "after a clock settle and the warm-up, K launches back to back between two HIP events on "
                  "the launch stream, each with only its stop event bound to its kernel's end (value, "
                  "ms_per_step; interval_ms_*: one kernel's end to the next one's), then K launches with "
                  "start and stop events bound to each kernel's dispatch by the library "
                  "(attn_fwd_ex_timed: kernel_ms_*, roofline.achieved); headline launches before the "
                  "timed ones: settle_launches + warmup",
    }
    checks = []
    sub = max(20, K // 4)
    if not args.no_bwd:
        extra["bwd"] = measure_backward(ta, pm, dev, stream, sub, 150.0, checks)
    if not args.no_ex:
        extra.update(measure_ex(ta, pm, dev, stream, sub, 150.0, checks))
        extra.update(measure_configs(ta, pm, dev, stream, sub, 150.0, checks))

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
    ok = True
    if args.cpu_seconds > 0:
        result["cpu_baseline"], extra["verify"] = cpu_leg(w, x_cpu, o_timed, lse_timed, args.cpu_seconds, checks)
        ok = extra["verify"]["pass"]
    print(json.dumps(result), flush=True)
    if not ok:
        print("bench.py: a measured output is outside the oracle bars (see extra.verify)", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
