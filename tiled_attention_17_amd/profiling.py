"""Profiling runs of the attention kernels and the summaries of their counter runs.

  python -m tiled_attention_17_amd.profiling run [--launches 5] [--copy-mib 1024]
      Enqueues one plain device-to-device copy of a known size (the
      calibration kernel for HBM byte counters) and then `launches` forward
      passes of the headline workload (B=2, H=16, N=4096, d=128, bf16).
      Meant to run under rocprofv3, e.g.
        rocprofv3 --pmc FETCH_SIZE -d OUT/pmc_fetch -o run --output-format csv \
            -- python -m tiled_attention_17_amd.profiling run

  python -m tiled_attention_17_amd.profiling run-set [--launches 3] [--copy-mib 1024]
      The calibration copy, then `launches` passes each of: the headline
      forward, the backward of the forward+backward workload, the d = 64
      forward (B=4 H=8 N=1024), the fp32 single-head forward, the decode
      forward (B=8 H=16, one query against 8192 keys, library key splits) and
      the MXFP8 forward at the headline shape. For counter runs of every
      kernel (see summarize-set).

  python -m tiled_attention_17_amd.profiling summarize-set --sq DIR --fetch DIR --write DIR
      Per kernel of a run-set: duration, shader clock (GRBM_GUI_ACTIVE over
      the duration), MFMA busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over the
      SIMD cycles), MFMA instructions, LDS bank-conflict cycles per LDS
      instruction, and HBM bytes (FETCH_SIZE + WRITE_SIZE, calibrated on the
      copy) with the achieved GB/s. Writes profiles/kernel_counters.md.

  python -m tiled_attention_17_amd.profiling summarize-bench --trace DIR --bench-line FILE --command CMD
      Reads the kernel trace (and --stats table) of a rocprofv3 run of
      bench.py together with the JSON line that run printed, and writes
      profiles/fwd_bf16_n4096_d128_kernel_stats.md: every kernel's calls and
      average duration, and the headline forward's timed launches picked out
      of the trace by launch order (bench.py launches the headline first:
      settle_launches + warmup untimed launches, then `steps` launches of the
      timed region, then `steps` launches with kernel-bound events), with
      their average duration and roofline fraction beside the line's.

  python -m tiled_attention_17_amd.profiling mfma-ceiling [--iters 1200] [--settle-ms 500] [--out-md FILE]
      Runs the matrix-core probe (libtattn_probe.so, csrc/mfma_ceiling.hip)
      in each of its modes on every CU, after a clock settle per mode, and
      writes a table of sustained bf16 TFLOP/s and shader clock: constant
      against random operands, with LDS operand reads and the softmax's
      vector work added, and the 16x16x32 shape.

  python -m tiled_attention_17_amd.profiling summarize --fetch DIR --write DIR [--stats DIR]
      Reads the counter CSVs of the two runs (FETCH_SIZE, WRITE_SIZE; KiB per
      dispatch), scales the forward kernel's figures by what the same counter
      reads for the copy of known size, and writes profiles/fwd_bf16_traffic.json
      (tagged with the kernel source digest, so bench.py stops reporting it once
      the kernel changes) and a short text summary.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FWD_KERNEL = "attn_fwd_bf16_pingpong_kernel"
KERNEL_SOURCES = [os.path.join(ROOT, "tiled_attention_17_amd", "csrc", f)
                  for f in ("attn_fwd.hip", "tile_common.h", "device_common.h")]


def source_digest():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def run(launches: int, copy_mib: int):
    import torch

    import tiled_attention_17_amd as ta
    from tiled_attention_17_amd.workloads import HEADLINE, make_inputs

    dev = torch.device("cuda:0")
    n = copy_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)  # calibration copy kernel: reads and writes exactly copy_mib MiB
    torch.cuda.synchronize()
    del src, dst
    w = HEADLINE
    x = {k: t.to(dev) for k, t in make_inputs(w).items()}
    o = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    for _ in range(launches):
        ta.attn_fwd(x["q"], x["k"], x["v"], w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    print(f"profiling run done: copy {copy_mib} MiB, {launches} forward launches of {w.name}", flush=True)


SET_SQ_COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES",
                   "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT"]
SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
XCDS = 8  # GRBM_GUI_ACTIVE reads the sum over the 8 XCDs (a 260 us dispatch: 3.76e6, 1.81 GHz each)


def run_set(launches: int, copy_mib: int):
    import torch

    import tiled_attention_17_amd as ta
    from tiled_attention_17_amd.workloads import EXTRA_WORKLOADS, HEADLINE, WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    n = copy_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)  # calibration copy kernel
    torch.cuda.synchronize()
    del src, dst

    def fwd(w, reps):
        x = {k: t.to(dev) for k, t in make_inputs(w).items()}
        for _ in range(reps):
            ta.attn_fwd(x["q"], x["k"], x["v"], w.scale)
        torch.cuda.synchronize()
        return x

    fwd(HEADLINE, launches)
    wb = WORKLOADS[4]
    xb = {k: t.to(dev) for k, t in make_inputs(wb).items()}
    ob, lb = ta.attn_fwd(xb["q"], xb["k"], xb["v"], wb.scale)
    for _ in range(launches):
        ta.attn_bwd(xb["q"], xb["k"], xb["v"], ob, xb["do"], lb, wb.scale)
    torch.cuda.synchronize()
    del xb, ob, lb
    fwd(WORKLOADS[1], launches)
    fwd(WORKLOADS[0], launches)
    wd = [w for w in EXTRA_WORKLOADS if w.name.startswith("decode")][0]
    xd = {k: t.to(dev) for k, t in make_inputs(wd).items()}
    s = ta.attn_fwd_ex_auto_splits(wd.B, wd.H, wd.Nq, wd.Nk, wd.d)
    for _ in range(launches):
        ta.attn_fwd_ex(xd["q"], xd["k"], xd["v"], wd.scale, num_splits=s)
    torch.cuda.synchronize()
    del xd
    x = {k: t.to(dev) for k, t in make_inputs(HEADLINE).items()}
    q8, qs = ta.attn_quantize_mxfp8(x["q"])
    k8, ks = ta.attn_quantize_mxfp8(x["k"])
    vt8, vts = ta.attn_quantize_mxfp8(x["v"], transpose=True)
    for _ in range(launches):
        ta.attn_fwd_mxfp8(q8, qs, k8, ks, vt8, vts, HEADLINE.scale)
    torch.cuda.synchronize()
    print(f"profiling set done: copy {copy_mib} MiB, {launches} launches per workload", flush=True)


def _short(name):
    name = name.split("(")[0].replace("void ", "").replace("tattn::", "")
    if name.startswith("_ZN5tattn23mx_quantize_rows"):
        return "mx_quantize_rows_kernel"
    if name.startswith("_ZN5tattn25mx_quantize_cols_t"):
        return "mx_quantize_cols_t_kernel"
    return name


def _by_dispatch(rows):
    """{dispatch id: {"kernel", "grid", "ns", counter: value summed over dimensions}}."""
    out = {}
    for r in rows:
        d = out.setdefault(r["Dispatch_Id"], {"kernel": _short(r["Kernel_Name"]),
                                              "grid": int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])),
                                              "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        c, v = r["Counter_Name"], float(r["Counter_Value"])
        # GRBM counters exist once per XCD and count the same clock: take the largest
        d[c] = max(d.get(c, 0.0), v) if c.startswith("GRBM_") else d.get(c, 0.0) + v
    return out


def summarize_set(sq_dir, fetch_dir, write_dir, copy_mib, out_md):
    copy_bytes = copy_mib * (1 << 20)
    sq = _by_dispatch(_counter_rows(sq_dir))
    fe = _by_dispatch(_counter_rows(fetch_dir))
    wr = _by_dispatch(_counter_rows(write_dir))

    def calib(disp, counter):
        vals = [d[counter] for d in disp.values() if "elementwise" in d["kernel"].lower()]
        if not vals:
            raise RuntimeError("no calibration copy in the counter run")
        return copy_bytes / max(vals)

    f_scale, w_scale = calib(fe, "FETCH_SIZE"), calib(wr, "WRITE_SIZE")

    def groups(disp):
        g = {}
        for d in disp.values():
            if "elementwise" in d["kernel"].lower():
                continue
            g.setdefault((d["kernel"], d["grid"]), []).append(d)
        return g

    gs, gf, gw = groups(sq), groups(fe), groups(wr)
    mean = lambda ds, k: sum(d.get(k, 0.0) for d in ds) / len(ds)
    lines = ["# Hardware counters per kernel (one MI355X)", "",
             "Three rocprofv3 runs of the same program (repo root, on the MI355X), each with counters the",
             "hardware collects in one pass:", "",
             "    rocprofv3 --pmc " + " ".join(SET_SQ_COUNTERS) + " \\",
             f"        -d {sq_dir} -o run --output-format csv \\",
             "        -- python3 tiled_attention_17_amd/profiling.py run-set",
             f"    rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run --output-format csv \\",
             "        -- python3 tiled_attention_17_amd/profiling.py run-set",
             f"    rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o run --output-format csv \\",
             "        -- python3 tiled_attention_17_amd/profiling.py run-set",
             f"    python3 -m tiled_attention_17_amd.profiling summarize-set --sq {sq_dir} \\",
             f"        --fetch {fetch_dir} --write {write_dir}", "",
             "Columns (means over a kernel's dispatches in the SQ run; counter runs serialize the",
             "dispatches, so the clock here is not the one of a sustained run, and for kernels of a few",
             "tens of microseconds the GRBM window also spans the dispatch itself, which inflates the",
             "clock and deflates the MFMA fraction):",
             f"- clock: GRBM_GUI_ACTIVE / {XCDS} (the counter sums the XCDs) / duration;",
             f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs), the fraction",
             "  of SIMD cycles the matrix cores worked;",
             "- MFMA insts: v_mfma instructions per dispatch (a 32x32x16 bf16 one is 32768 FLOPs);",
             "- LDS conflict: SQ_LDS_BANK_CONFLICT cycles per LDS instruction (SQ_INSTS_LDS);",
             f"- HBM: FETCH_SIZE + WRITE_SIZE scaled so that a {copy_mib} MiB copy reads and writes {copy_mib} MiB "
             f"(x{f_scale:.1f} and x{w_scale:.1f} bytes per unit), and that over the duration.", "",
             "| kernel | workgroups | dispatches | us | clock GHz | MFMA busy | MFMA insts | LDS conflict / inst "
             "| HBM MB | HBM GB/s |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for key, ds in gs.items():
        ns = mean(ds, "ns")
        gui = mean(ds, "GRBM_GUI_ACTIVE") / XCDS  # cycles of one XCD
        clock = gui / ns if ns else 0.0
        busy = mean(ds, "SQ_VALU_MFMA_BUSY_CYCLES") / (gui * SIMDS) if gui else 0.0
        lds = mean(ds, "SQ_INSTS_LDS")
        conf = mean(ds, "SQ_LDS_BANK_CONFLICT") / lds if lds else 0.0
        hbm = None
        if key in gf and key in gw:
            hbm = mean(gf[key], "FETCH_SIZE") * f_scale + mean(gw[key], "WRITE_SIZE") * w_scale
        lines.append(f"| {key[0]} | {key[1]} | {len(ds)} | {ns / 1e3:.1f} | {clock:.2f} | {100 * busy:.1f} % "
                     f"| {mean(ds, 'SQ_INSTS_MFMA'):.3g} | {conf:.3f} "
                     f"| {'' if hbm is None else f'{hbm / 1e6:.1f}'} "
                     f"| {'' if hbm is None or not ns else f'{hbm / ns:.0f}'} |")
    lines += ["",
              "Cross-checks: MFMA insts x 32768 FLOPs equals the algorithmic 4 B H N^2 d of the headline",
              "forward (no redundant matrix work); MFMA busy x clock / 2.4 GHz x 2.5 PFLOP/s reproduces",
              "its measured rate; the bf16 kernels' LDS layouts (swizzled K, V^T, Q/dO tiles and their",
              "transposed reads) show no bank-conflict cycles (the one-query kernel's LDS traffic is its",
              "cross-lane shuffles and the end-of-sweep merge of its waves, once per workgroup); HBM bytes",
              "of the headline forward match its algorithmic bytes, and decode runs near the HBM rate."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_rows(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter):
    """{(dispatch id, kernel name): value} for one counter (summed over dimensions)."""
    out = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (r.get("Dispatch_Id"), r.get("Kernel_Name"))
        out[key] = out.get(key, 0.0) + float(r["Counter_Value"])
    return out


def _split(vals):
    copies = [v for (d, k), v in vals.items() if FWD_KERNEL not in k and "elementwise" in k.lower()]
    fwd = [v for (d, k), v in vals.items() if FWD_KERNEL in k]
    return copies, fwd


def summarize(fetch_dir, write_dir, stats_dir, copy_mib, out_json, out_txt):
    from tiled_attention_17_amd import perfmodel as pm
    from tiled_attention_17_amd.workloads import HEADLINE as w

    copy_bytes = copy_mib * (1 << 20)
    fc, ff = _split(_per_dispatch(_counter_rows(fetch_dir), "FETCH_SIZE"))
    wc, wf = _split(_per_dispatch(_counter_rows(write_dir), "WRITE_SIZE"))
    if not (fc and ff and wc and wf):
        raise RuntimeError("missing copy or forward dispatches in the counter runs")
    # Scale so that the copy reads and writes exactly copy_bytes.
    f_scale = copy_bytes / max(fc)
    w_scale = copy_bytes / max(wc)
    fetch = sum(ff) / len(ff) * f_scale
    write = sum(wf) / len(wf) * w_scale
    algo = pm.attn_fwd_bytes(w.B, w.H, w.N, w.d, 2)
    res = {
        "kernel": FWD_KERNEL,
        "workload": w.name,
        "source_sha256": source_digest(),
        "copy_calibration_bytes": copy_bytes,
        "fetch_size_copy_raw_kib": max(fc),
        "write_size_copy_raw_kib": max(wc),
        "fetch_scale_bytes_per_unit": f_scale,
        "write_scale_bytes_per_unit": w_scale,
        "fetch_bytes_per_launch": fetch,
        "write_bytes_per_launch": write,
        "bytes_per_launch": fetch + write,
        "algorithmic_bytes_per_launch": algo,
        "traffic_over_algorithmic": (fetch + write) / algo,
    }
    with open(out_json, "w") as f:
        json.dump(res, f, indent=2)
    lines = [f"# HBM traffic of {FWD_KERNEL} on {w.name}", "",
             "Counters FETCH_SIZE and WRITE_SIZE (one rocprofv3 --pmc run each), scaled by the",
             f"same counters on a {copy_mib} MiB device-to-device copy. Commands (repo root):", "",
             f"    rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run --output-format csv \\",
             "        -- python3 tiled_attention_17_amd/profiling.py run",
             f"    rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o run --output-format csv \\",
             "        -- python3 tiled_attention_17_amd/profiling.py run",
             f"    python3 -m tiled_attention_17_amd.profiling summarize --fetch {fetch_dir} \\",
             f"        --write {write_dir}", "",
             f"The copy reads {copy_bytes} bytes and writes as many; the counters read "
             f"{max(fc):.0f} and {max(wc):.0f} units for it, which gives the scale factors below.", ""]
    for k, v in res.items():
        lines.append(f"- {k}: {v}")
    if stats_dir:
        lines.append("")
        lines.append("Kernel stats of the same program:")
        for f in glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True):
            lines.extend(open(f).read().strip().splitlines())
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(res, indent=2))


def _csv_rows(d, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_bench(trace_dir, bench_line, cmd, out_md):
    """Kernel-trace summary of one bench.py run, with the headline's timed launches picked out."""
    with open(bench_line) as f:
        line = next(json.loads(s) for s in f if s.startswith("{"))
    ex = line["extra"]
    steps, warm = line["steps"], line["warmup"]
    untimed = ex["settle_launches"] + warm
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    disp = sorted(((int(r["Dispatch_Id"]), _short(r["Kernel_Name"]),
                    int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in trace))
    fwd = [ns for _, k, ns in disp if k.startswith(FWD_KERNEL)]
    region = fwd[untimed:untimed + steps]
    timed = fwd[untimed + steps:untimed + 2 * steps]
    if len(timed) != steps:
        raise SystemExit(f"trace holds {len(fwd)} forward launches, fewer than {untimed} + 2 * {steps}")
    flops = 4 * line["config"]["B"] * line["config"]["H"] * line["config"]["N"] ** 2 * line["config"]["d"]
    peak = line["roofline"]["peak"] * 1e12
    avg_us = sum(timed) / steps / 1e3
    region_us = sum(region) / steps / 1e3
    srt = sorted(timed)
    frac_trace = flops / (avg_us * 1e-6) / peak
    groups = {}
    for _, k, ns in disp:
        g = groups.setdefault(k, [0, 0, None, 0])
        g[0] += 1
        g[1] += ns
        g[2] = ns if g[2] is None else min(g[2], ns)
        g[3] = max(g[3], ns)
    lines = [
        f"# Kernel trace of the benchmark command: headline forward {line['config']['workload']}", "",
        "Command (repo root, on the MI355X):", "",
        f"    {cmd}", "",
        "## Headline forward: the timed launches", "",
        f"bench.py launched the headline forward {ex['settle_launches']} times to settle the clock "
        f"({ex['settle_ms']:.0f} ms of GPU time), {warm} warm-up times, then {steps} times back to back "
        f"in the timed region (forward launches {untimed + 1}..{untimed + steps} of the trace: `value`, "
        f"`ms_per_step`), then {steps} times with start and stop events bound to each kernel (launches "
        f"{untimed + steps + 1}..{untimed + 2 * steps}: `roofline.achieved`). The headline is the first "
        "workload bench.py runs.", "",
        "| figure | kernel trace | bench.py line (HIP events) |",
        "|---|---|---|",
        f"| timed region: average duration / time per launch | {region_us:.1f} us | "
        f"{ex.get('interval_ms_mean', float('nan')) * 1e3:.1f} us from one kernel's end to the next "
        f"one's; {line['ms_per_step'] * 1e3:.1f} us per step |",
        f"| kernel-bound events: average duration | {avg_us:.1f} us | {ex['kernel_ms_mean'] * 1e3:.1f} us |",
        f"| median duration | {srt[steps // 2] / 1e3:.1f} us | {ex['kernel_ms_median'] * 1e3:.1f} us |",
        f"| min duration | {srt[0] / 1e3:.1f} us | {ex['kernel_ms_min'] * 1e3:.1f} us |",
        f"| TFLOP/s at 4·B·H·N²·d = {flops / 1e9:.1f} GFLOP | {flops / (avg_us * 1e-6) / 1e12:.1f} | "
        f"{line['roofline']['achieved']:.1f} |",
        f"| roofline frac (peak {line['roofline']['peak']:.0f} TFLOP/s) | {frac_trace:.4f} | "
        f"{line['roofline']['frac']:.4f} |", "",
        f"Line vs trace: {100.0 * (line['roofline']['frac'] / frac_trace - 1):+.1f} % (the bound start "
        "event marks the end of a marker command just before the kernel's dispatch).", "",
        "## Every kernel of the run (rocprofv3 kernel trace; durations in us)", "",
        "| kernel | calls | average | min | max |", "|---|---|---|---|---|"]
    for k, (n, tot, mn, mx) in sorted(groups.items(), key=lambda kv: -kv[1][1]):
        lines.append(f"| {k} | {n} | {tot / n / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} |")
    lines += ["", "The forward kernel's average over all its calls also holds the settle launches, the "
              "warm-up, and the causal, query-shard and long-sequence launches (other shapes), so only "
              "the timed window above compares with the line.", "",
              "Bench line of the same run:", "", "    " + json.dumps({k: line[k] for k in (
                  "value", "ms_per_step", "steps", "warmup", "roofline")})]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:20]))


PROBE_MODES = [
    (0, "32x32x16, constant operands"),
    (1, "32x32x16, random operands"),
    (3, "32x32x16, random, A read from LDS"),
    (5, "32x32x16, random, + one softmax element per MFMA"),
    (7, "32x32x16, random, LDS A + softmax element"),
    (9, "16x16x32 (two per unit), random operands"),
    (15, "16x16x32, random, LDS A + softmax element"),
    (19, "LDS reads alone (no MFMA)"),
    (21, "softmax elements alone (no MFMA)"),
    (33, "32x32x16, random, B shared by 4 consecutive MFMAs"),
    (65, "32x32x16, random, A shared by 4 consecutive MFMAs"),
    (97, "32x32x16, random, A and B shared by 4 consecutive MFMAs"),
    (129, "32x32x16, random, A shared by 2 consecutive MFMAs"),
    (135, "32x32x16, random, LDS A read per 2 MFMAs + softmax element"),
    (71, "32x32x16, random, LDS A read per 4 MFMAs + softmax element"),
]


def mfma_ceiling(iters, settle_ms, out_md, command):
    """Sustained matrix-core rate and shader clock per probe mode (see csrc/mfma_ceiling.hip)."""
    import ctypes
    import time

    import torch

    from tiled_attention_17_amd.build import LIB_PROBE

    if not os.path.exists(LIB_PROBE):
        raise RuntimeError(f"{LIB_PROBE} is not built (tiled_attention_17_amd/build.py --probe)")
    lib = ctypes.CDLL(LIB_PROBE)
    lib.tattn_probe_mfma_ceiling.restype = ctypes.c_int
    lib.tattn_probe_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    props = torch.cuda.get_device_properties(0)
    grid = props.multi_processor_count
    out = torch.zeros(grid * 8 * 2, dtype=torch.int64, device="cuda")
    sink = torch.zeros(grid * 512, dtype=torch.float32, device="cuda")
    g = torch.Generator().manual_seed(1)
    rnd_vecs = grid * 512 * 16
    rnd = torch.randn(rnd_vecs * 8, generator=g).to(torch.bfloat16).cuda()  # N(0, 1) bf16, 8 per 16-byte word
    st = torch.cuda.current_stream().cuda_stream

    def launch(mode):
        r = lib.tattn_probe_mfma_ceiling(mode, out.data_ptr(), sink.data_ptr(), rnd.data_ptr(), rnd_vecs, grid,
                                         iters, st)
        if r != 0:
            raise RuntimeError(f"probe mode {mode}: status {r}")

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rows = []
    for mode, desc in PROBE_MODES:
        t_end = time.time() + settle_ms / 1e3
        while time.time() < t_end:
            for _ in range(10):
                launch(mode)
            torch.cuda.synchronize()
        ev[0].record()
        for _ in range(10):
            launch(mode)
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) / 10 * 1e3
        o = out.view(-1, 2).cpu().double()
        clock = (o[:, 0] / o[:, 1]).median().item() * 0.1  # shader ticks per 100 MHz tick -> GHz
        tf = 0.0 if mode & 16 else grid * 8 * iters * 8 * 32768 / (us * 1e-6) / 1e12
        rows.append((mode, desc, us, clock, tf))
        print(f"mode {mode:2d} {desc:48s} {us:8.1f} us  clock {clock:5.2f} GHz  {tf:7.1f} TFLOP/s", flush=True)
    lines = [
        "# Sustained bf16 matrix-core rate and shader clock (one MI355X)",
        "",
        "Measurement probe `tiled_attention_17_amd/csrc/mfma_ceiling.hip` (library `libtattn_probe.so`), one",
        f"512-thread workgroup on each of the {grid} CUs, two waves per SIMD, {iters} iterations of 8 units of",
        "32768 FLOPs per wave, each mode after a clock settle of "
        f"{settle_ms} ms; time from HIP events over 10 launches, clock",
        "from the waves' `s_memtime` / `s_memrealtime` ticks. Random operands are N(0, 1) in bf16, as the",
        "attention workloads' inputs; the softmax element is one FMA, one exp2, one add and half a bf16 pack.",
        "The LDS modes keep two operand reads in flight per wave, so part of their drop is read latency;",
        "their clocks show what the reads add to the power.",
        "",
        "Command (repo root, on the MI355X):",
        "",
        f"    {command}",
        "",
        "| mode | work | us per launch | clock GHz | TFLOP/s | % of 2.5 PFLOP/s |",
        "|---|---|---|---|---|---|",
    ]
    for mode, desc, us, clock, tf in rows:
        pct = f"{tf / 2500 * 100:.1f} %" if tf else "-"
        tfs = f"{tf:.0f}" if tf else "-"
        lines.append(f"| {mode} | {desc} | {us:.1f} | {clock:.2f} | {tfs} | {pct} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", out_md)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--launches", type=int, default=5)
    r.add_argument("--copy-mib", type=int, default=1024)
    rs = sub.add_parser("run-set")
    rs.add_argument("--launches", type=int, default=3)
    rs.add_argument("--copy-mib", type=int, default=1024)
    ss = sub.add_parser("summarize-set")
    ss.add_argument("--sq", required=True)
    ss.add_argument("--fetch", required=True)
    ss.add_argument("--write", required=True)
    ss.add_argument("--copy-mib", type=int, default=1024)
    ss.add_argument("--out-md", default=os.path.join(ROOT, "profiles", "kernel_counters.md"))
    sb = sub.add_parser("summarize-bench")
    sb.add_argument("--trace", required=True)
    sb.add_argument("--bench-line", required=True)
    sb.add_argument("--command", required=True)
    sb.add_argument("--out-md", default=os.path.join(ROOT, "profiles", "fwd_bf16_n4096_d128_kernel_stats.md"))
    mc = sub.add_parser("mfma-ceiling")
    mc.add_argument("--iters", type=int, default=1200)
    mc.add_argument("--settle-ms", type=int, default=500)
    mc.add_argument("--out-md", default=os.path.join(ROOT, "profiles", "mfma_ceiling_bf16.md"))
    mc.add_argument("--command", default="python3 -m tiled_attention_17_amd.profiling mfma-ceiling")
    s = sub.add_parser("summarize")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--stats")
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--out-json", default=os.path.join(ROOT, "profiles", "fwd_bf16_traffic.json"))
    s.add_argument("--out-txt", default=os.path.join(ROOT, "profiles", "fwd_bf16_n4096_d128_traffic.md"))
    a = ap.parse_args()
    if a.cmd == "run":
        run(a.launches, a.copy_mib)
    elif a.cmd == "run-set":
        run_set(a.launches, a.copy_mib)
    elif a.cmd == "summarize-bench":
        summarize_bench(a.trace, a.bench_line, a.command, a.out_md)
    elif a.cmd == "mfma-ceiling":
        mfma_ceiling(a.iters, a.settle_ms, a.out_md, a.command)
    elif a.cmd == "summarize-set":
        summarize_set(a.sq, a.fetch, a.write, a.copy_mib, a.out_md)
    else:
        summarize(a.fetch, a.write, a.stats, a.copy_mib, a.out_json, a.out_txt)


if __name__ == "__main__":
    main()
