"""The matrix-core measurement probe (csrc/mfma_ceiling.hip, libtattn_probe.so).

It is a measurement tool beside the attention library, not part of the path:
these tests check that it is built, exports its entry point and rejects bad
arguments on the host, and (on a GPU) that one short run reports a plausible
clock and rate.
"""

import ctypes
import os

import pytest

from tiled_attention_17_amd.build import LIB_PROBE


def _lib():
    if not os.path.exists(LIB_PROBE):
        pytest.skip("libtattn_probe.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PROBE)
    lib.tattn_probe_mfma_ceiling.restype = ctypes.c_int
    lib.tattn_probe_mfma_ceiling.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


def test_probe_rejects_bad_arguments_on_the_host():
    lib = _lib()
    one = ctypes.c_int64(0)
    p = ctypes.addressof(one)
    assert lib.tattn_probe_mfma_ceiling(1, None, p, p, 1, 1, 1, None) == 1  # no output buffer
    assert lib.tattn_probe_mfma_ceiling(1, p, p, p, 0, 1, 1, None) == 1    # empty operand buffer
    assert lib.tattn_probe_mfma_ceiling(1, p, p, p, 1, 0, 1, None) == 1    # no workgroup
    assert lib.tattn_probe_mfma_ceiling(2, p, p, p, 1, 1, 1, None) == 1    # unknown mode


@pytest.mark.gpu
def test_probe_short_run_is_plausible():
    import torch

    lib = _lib()
    grid, iters = torch.cuda.get_device_properties(0).multi_processor_count, 200
    out = torch.zeros(grid * 16, dtype=torch.int64, device="cuda")
    sink = torch.zeros(grid * 512, dtype=torch.float32, device="cuda")
    rnd = torch.randn(grid * 512 * 16 * 8).to(torch.bfloat16).cuda()
    st = torch.cuda.current_stream().cuda_stream
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for _ in range(3):
        assert lib.tattn_probe_mfma_ceiling(7, out.data_ptr(), sink.data_ptr(), rnd.data_ptr(), grid * 512 * 16,
                                            grid, iters, st) == 0
    ev[0].record()
    assert lib.tattn_probe_mfma_ceiling(7, out.data_ptr(), sink.data_ptr(), rnd.data_ptr(), grid * 512 * 16,
                                        grid, iters, st) == 0
    ev[1].record()
    torch.cuda.synchronize()
    o = out.view(-1, 2).cpu().double()
    assert torch.all(o > 0)
    clock = (o[:, 0] / o[:, 1]).median().item() * 0.1
    assert 0.5 < clock < 3.0, clock
    tflops = grid * 8 * iters * 8 * 32768 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12
    assert 50 < tflops < 2600, tflops
    assert torch.isfinite(sink).all()
