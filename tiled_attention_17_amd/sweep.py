"""Matrix-product size sweep on one MI355X: throughput against size and wave quantization.

The CS336 Lecture 5 notes (§6.2) show matmul throughput falling off a cliff
when the number of output tiles passes a whole number of rounds over the
compute units (256 x 128 tiles on 108 SMs: 1792^2 gives 98 tiles, one round;
1793^2 gives 120, a second round of 12). This module measures the same
effect for attn_matmul_nt on MI355X: one workgroup per 128 x 128 tile of C,
two resident workgroups per compute unit, 256 compute units, so one round
holds 512 tiles. For each size it prints the measured TFLOP/s next to the
model's prediction (tiles / (rounds * 512), the fraction of the last round's
slots that hold work), and torch.matmul (hipBLASLt) on the same operands
for context.

Usage: python -m tiled_attention_17_amd.sweep [--k 4096] [--sizes 1024,1025,...]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TILE = 128
WG_PER_CU = 2

# Sizes on both sides of whole rounds of 512 tiles (tiles = ceil(S/128)^2):
# 2816 -> 484 (one round), 2944 -> 529 (two), 4096 -> 1024 (two, full),
# 4097 -> 1089 (three), 5760/5761, 8064/8065 ...
DEFAULT_SIZES = [1024, 1536, 2048, 2560, 2816, 2880, 2944, 3072, 3584, 3968, 4096, 4097, 4224,
                 4608, 5120, 5632, 5760, 5761, 6144, 7168, 8064, 8065, 8192]


def model(size, cus):
    tiles = math.ceil(size / TILE) ** 2
    slots = cus * WG_PER_CU
    rounds = math.ceil(tiles / slots)
    return tiles, rounds, tiles / (rounds * slots)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--k", type=int, default=4096)
    ap.add_argument("--sizes", type=str, default=",".join(map(str, DEFAULT_SIZES)))
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--no-library", action="store_true", help="skip the torch.matmul column")
    args = ap.parse_args()

    import torch

    import tiled_attention_17_amd as ta
    from tiled_attention_17_amd import perfmodel as pm

    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    st = torch.cuda.current_stream(dev)
    peak = pm.MI355X_PEAK_FLOPS["bf16"] / 1e12
    g = torch.Generator(device="cpu").manual_seed(11)

    def tms(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(args.iters):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.iters

    # warm the clock up (it ramps over tens of ms under load)
    a = torch.randn((4096, args.k), generator=g).to(torch.bfloat16).to(dev)
    for _ in range(200):
        ta.attn_matmul_nt(a, a)
    torch.cuda.synchronize()

    print(f"# attn_matmul_nt, C = A B^T, bf16, K = {args.k}, {cus} CUs, 128 x 128 tiles, "
          f"{WG_PER_CU} workgroups per CU", flush=True)
    print(f"# {'size':>6} {'tiles':>6} {'rounds':>6} {'model':>6} {'us':>9} {'TFLOP/s':>8} {'%peak':>6}"
          f" {'lib TFLOP/s':>11}", flush=True)
    for size in [int(s) for s in args.sizes.split(",")]:
        a = torch.randn((size, args.k), generator=g).to(torch.bfloat16).to(dev)
        b = torch.randn((size, args.k), generator=g).to(torch.bfloat16).to(dev)
        c = torch.empty((size, size), dtype=torch.bfloat16, device=dev)
        ms = tms(lambda: ta.attn_matmul_nt(a, b, out=c))
        fl = pm.matmul_flops(size, args.k, size)
        tiles, rounds, eff = model(size, cus)
        lib = None
        if not args.no_library:
            bt = b.t()
            lms = tms(lambda: torch.matmul(a, bt))
            lib = fl / (lms * 1e-3) / 1e12
        tf = fl / (ms * 1e-3) / 1e12
        print(f"  {size:6d} {tiles:6d} {rounds:6d} {eff:6.3f} {ms * 1e3:9.1f} {tf:8.1f} {100 * tf / peak:6.1f}"
              f" {lib if lib is not None else float('nan'):11.1f}", flush=True)
        print(json.dumps({"size": size, "k": args.k, "tiles": tiles, "rounds": rounds, "model_fill": eff,
                          "us": ms * 1e3, "tflops": tf, "pct_of_bf16_dense_peak": 100 * tf / peak,
                          "torch_matmul_tflops": lib}), flush=True)
        del a, b, c


if __name__ == "__main__":
    main()
