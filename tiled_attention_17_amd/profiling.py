"""Profiling driver for the forward kernel and the summary of its counter runs.

  python -m tiled_attention_17_amd.profiling run [--launches 5] [--copy-mib 1024]
      Enqueues one plain device-to-device copy of a known size (the
      calibration kernel for HBM byte counters) and then `launches` forward
      passes of the headline workload (B=2, H=16, N=4096, d=128, bf16).
      Meant to run under rocprofv3, e.g.
        rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o run --output-format csv \
            -- python -m tiled_attention_17_amd.profiling run

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
             "    rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc_fetch -o run --output-format csv \\",
             "        -- python3 tiled_attention_17_amd/profiling.py run",
             "    rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc_write -o run --output-format csv \\",
             "        -- python3 tiled_attention_17_amd/profiling.py run",
             "    python3 -m tiled_attention_17_amd.profiling summarize --fetch gpurun_out/pmc_fetch \\",
             "        --write gpurun_out/pmc_write", "",
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


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--launches", type=int, default=5)
    r.add_argument("--copy-mib", type=int, default=1024)
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
    else:
        summarize(a.fetch, a.write, a.stats, a.copy_mib, a.out_json, a.out_txt)


if __name__ == "__main__":
    main()
