"""Build the HIP library in-tree for gfx950 with hipcc.

libtiledattn.so is the library. libtiledattn_ordered.so is the same sources
built with TATTN_ORDERED_LDS_DMA: every LDS transfer the kernels order by
hand goes through the form the compiler orders, with an extra wait and
barrier where a staged tile is published. It is a debug build for parity
runs (the binding loads it when TILED_ATTN_LIBRARY=ordered), never the
measured one. libtattn_probe.so is a measurement probe of the chip's
sustained matrix-core rate (profiling.py mfma-ceiling), apart from the
attention path.
"""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtiledattn.so")
LIB_ORDERED = os.path.join(PKG, "libtiledattn_ordered.so")
# measurement probe (profiling.py mfma-ceiling), never loaded by the attention path
LIB_PROBE = os.path.join(PKG, "libtattn_probe.so")
PROBE_SOURCES = ["mfma_ceiling.hip"]
SOURCES = ["api.cpp", "attn_fwd.hip", "attn_bwd.hip", "matmul.hip", "attn_fp8.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def build(verbose: bool = False, ordered_lds_dma: bool = False, probe: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = LIB_PROBE if probe else (LIB_ORDERED if ordered_lds_dma else LIB)
    tmp = out + ".tmp"
    defs = ["-DTATTN_ORDERED_LDS_DMA"] if ordered_lds_dma else []
    sources = PROBE_SOURCES if probe else SOURCES
    cmd = [hipcc, *FLAGS, *defs, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, ordered_lds_dma="--ordered-lds-dma" in sys.argv,
                probe="--probe" in sys.argv))
