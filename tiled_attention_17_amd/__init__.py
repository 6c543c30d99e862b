"""Fused softmax attention for MI355X (gfx950): Python binding of libtiledattn.so.

The functions here only marshal arguments: they check tensor metadata,
allocate outputs with torch (device memory), and call the C-ABI entry points
of the same names declared in include/tiled_attn.h on the current HIP
stream. Every step of the computation runs in the library's HIP kernels;
there is no fallback. If the library has not been built, calling any of them
raises immediately.
"""

from __future__ import annotations

import contextlib
import ctypes
import math
import os

__all__ = ["attn_fwd", "attn_fwd_ex", "attn_fwd_ex_timed", "attn_fwd_ex_workspace_bytes", "attn_fwd_ex_auto_splits",
           "attn_merge", "attn_bwd", "attn_bwd_ex", "attn_bwd_workspace_bytes", "attn_matmul_nt",
           "attn_quantize_mxfp8", "attn_fwd_mxfp8", "attn_bwd_ex_noalloc", "ATTN_NOALLOC_MAX_ROWS",
           "library", "AttnError",
           "ATTN_BF16", "ATTN_FP32", "ATTN_MASK_NONE", "ATTN_MASK_CAUSAL", "LIB_PATH"]

# TILED_ATTN_LIBRARY=ordered selects the debug build whose LDS transfers are
# all ordered by the compiler (see build.py); the default is the release build.
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libtiledattn_ordered.so" if os.environ.get("TILED_ATTN_LIBRARY") == "ordered"
                        else "libtiledattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARGUMENT, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_BF16, ATTN_FP32 = 0, 1
ATTN_MASK_NONE, ATTN_MASK_CAUSAL = 0, 1
ATTN_NOALLOC_MAX_ROWS = 1 << 22

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def library():
    """The loaded libtiledattn.so (ctypes), loading it on first use."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run __graft_entry__.build() or python tiled_attention_17_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_vp, c_f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.attn_version.restype = ctypes.c_int
    lib.attn_version.argtypes = []
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_f,
                             ctypes.c_int, c_vp]
    lib.attn_fwd_ex_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_ex_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, ctypes.c_int]
    lib.attn_fwd_ex_auto_splits.restype = c_i64
    lib.attn_fwd_ex_auto_splits.argtypes = [c_i64, c_i64, c_i64, c_i64, c_i64, ctypes.c_int]
    lib.attn_fwd_ex.restype = ctypes.c_int
    lib.attn_fwd_ex.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_f,
                                ctypes.c_int, c_i64, c_vp, ctypes.c_size_t, ctypes.c_int, c_vp]
    lib.attn_fwd_ex_timed.restype = ctypes.c_int
    lib.attn_fwd_ex_timed.argtypes = lib.attn_fwd_ex.argtypes + [c_vp, c_vp]
    lib.attn_merge.restype = ctypes.c_int
    lib.attn_merge.argtypes = [c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp,
                               ctypes.c_int, c_vp]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd_workspace_bytes.argtypes = [c_i64, c_i64, c_i64, c_i64, ctypes.c_int]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_bwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                             ctypes.c_size_t, c_i64, c_i64, c_i64, c_i64, c_f, ctypes.c_int, c_vp]
    lib.attn_quantize_mxfp8.restype = ctypes.c_int
    lib.attn_quantize_mxfp8.argtypes = [c_vp, c_i64, c_i64, c_i64, ctypes.c_int, c_vp, c_vp, ctypes.c_int,
                                        c_vp]
    lib.attn_fwd_mxfp8.restype = ctypes.c_int
    lib.attn_fwd_mxfp8.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64,
                                   c_i64, c_f, c_vp]
    lib.attn_matmul_nt.restype = ctypes.c_int
    lib.attn_matmul_nt.argtypes = [c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, ctypes.c_int, c_vp]
    lib.attn_bwd_ex_noalloc.restype = ctypes.c_int
    lib.attn_bwd_ex_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_i64, c_i64, c_i64, c_i64, c_i64, c_f, ctypes.c_int,
                                        ctypes.c_int, c_vp]
    lib.attn_bwd_ex.restype = ctypes.c_int
    lib.attn_bwd_ex.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                ctypes.c_size_t, c_i64, c_i64, c_i64, c_i64, c_i64, c_f, ctypes.c_int,
                                ctypes.c_int, c_vp]
    _lib = lib
    return lib


def _check(status: int):
    if status != ATTN_OK:
        lib = library()
        msg = lib.attn_last_error().decode() or lib.attn_status_string(status).decode()
        raise AttnError(status, msg)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _shape4(name, t, shape=None, dtype=None, device=None):
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, N, d], got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device, stream):
    import torch
    if stream is None:
        # torch's raw current-stream query skips building a Stream object
        # (a few microseconds, which matter for launches of a few microseconds).
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            index = device.index if device.index is not None else torch.cuda.current_device()
            return ctypes.c_void_p(raw(index))
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_device(device):
    """torch.cuda.device(device), or nothing to do when it is already current."""
    import torch
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def attn_fwd(q, k, v, scale=None, *, out=None, lse=None, stream=None):
    """O, LSE = attention forward of [B, H, N, d] tensors q, k, v (see attn_fwd in tiled_attn.h).

    scale defaults to 1/sqrt(d). Returns (O like q, LSE float32 [B, H, N]).
    """
    import torch
    lib = library()
    _shape4("q", q)
    shape, dt, dev = tuple(q.shape), q.dtype, q.device
    _shape4("k", k, shape, dt, dev)
    _shape4("v", v, shape, dt, dev)
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    B, H, N, d = shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shape4("out", out, shape, dt, dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _lse_out(lse, (B, H, N), dev)
    with _on_device(dev):
        st = lib.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, N, d, float(scale), _dtype_code(q), _stream(dev, stream))
    _check(st)
    return out, lse


def attn_fwd_ex_workspace_bytes(B, H, Nq, Nk, d, num_splits, dtype_code=ATTN_BF16):
    return int(library().attn_fwd_ex_workspace_bytes(B, H, Nq, Nk, d, num_splits, dtype_code))


def attn_fwd_ex_auto_splits(B, H, Nq, Nk, d, dtype_code=ATTN_BF16):
    """Key splits attn_fwd_ex uses with num_splits=0 on the current device."""
    return int(library().attn_fwd_ex_auto_splits(B, H, Nq, Nk, d, dtype_code))


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def attn_fwd_ex(q, k, v, scale=None, *, causal=False, num_splits=1, out=None, lse=None,
                workspace=None, stream=None):
    """O, LSE of q [B, H, Nq, d] against k, v [B, H, Nk, d] (see attn_fwd_ex in tiled_attn.h).

    causal: query i sees key j iff j <= i + Nk - Nq. num_splits: 1 = one pass,
    2..128 = that many key ranges merged afterwards, 0 = the library's choice.
    The split workspace is allocated here unless given.
    """
    return _fwd_ex(q, k, v, scale, causal, num_splits, out, lse, workspace, stream, None)


def attn_fwd_ex_timed(q, k, v, start, stop, scale=None, *, causal=False, num_splits=1, out=None,
                      lse=None, workspace=None, stream=None):
    """attn_fwd_ex that binds two timing events to its attention kernel (see attn_fwd_ex_timed).

    start, stop: torch.cuda.Event(enable_timing=True) or None. After the
    stream has reached the call, start.elapsed_time(stop) is the attention
    kernel's own execution time in ms. torch creates an event's HIP handle on
    its first record, so an event not yet recorded is recorded once here,
    on the same stream, before the call.
    """
    return _fwd_ex(q, k, v, scale, causal, num_splits, out, lse, workspace, stream, (start, stop))


def _event_handle(ev, device, stream):
    import torch
    if ev is None:
        return None
    if not isinstance(ev, torch.cuda.Event):
        raise TypeError(f"expected a torch.cuda.Event or None, got {type(ev).__name__}")
    if not ev.cuda_event:
        ev.record(stream if stream is not None else torch.cuda.current_stream(device))
    return ev.cuda_event


def _fwd_ex(q, k, v, scale, causal, num_splits, out, lse, workspace, stream, events):
    import torch
    lib = library()
    _shape4("q", q)
    dt, dev = q.dtype, q.device
    B, H, Nq, d = q.shape
    _shape4("k", k, None, dt, dev)
    Nk = k.shape[2]
    _shape4("k", k, (B, H, Nk, d), dt, dev)
    _shape4("v", v, (B, H, Nk, d), dt, dev)
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _shape4("out", out, (B, H, Nq, d), dt, dev)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    _lse_out(lse, (B, H, Nq), dev)
    code = _dtype_code(q)
    mask = ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE
    with _on_device(dev):
        # num_splits = 0 goes through as 0: the library's own choice, whose
        # workspace attn_fwd_ex_workspace_bytes(..., 0) reports.
        splits = num_splits
        need = attn_fwd_ex_workspace_bytes(B, H, Nq, Nk, d, splits, code)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        fwd_args = (q.data_ptr(), _ptr(k), _ptr(v), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                    float(scale), mask, splits, _ptr(workspace), ws_bytes, code, _stream(dev, stream))
        if events is None:
            st = lib.attn_fwd_ex(*fwd_args)
        else:
            st = lib.attn_fwd_ex_timed(*fwd_args, _event_handle(events[0], dev, stream),
                                       _event_handle(events[1], dev, stream))
    _check(st)
    return out, lse


def attn_merge(o_parts, lse_parts, *, dtype=None, out=None, lse=None, stream=None):
    """Merge fp32 partial results o_parts [P, B, H, N, d], lse_parts [P, B, H, N] (see attn_merge)."""
    import torch
    lib = library()
    if o_parts.dim() != 5 or o_parts.dtype != torch.float32 or not o_parts.is_contiguous():
        raise ValueError("o_parts must be a contiguous float32 [P, B, H, N, d] tensor")
    P, B, H, N, d = o_parts.shape
    if tuple(lse_parts.shape) != (P, B, H, N) or lse_parts.dtype != torch.float32 \
            or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be a contiguous float32 [P, B, H, N] tensor")
    dev = o_parts.device
    if lse_parts.device != dev:
        raise ValueError(f"lse_parts is on {lse_parts.device}, expected {dev}")
    dtype = torch.bfloat16 if dtype is None else dtype
    if out is not None:
        _shape4("out", out, (B, H, N, d), dtype, dev)
    if lse is not None:
        _lse_out(lse, (B, H, N), dev)
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    if out is None:
        out = torch.empty((B, H, N, d), dtype=dtype, device=dev)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    with _on_device(dev):
        st = lib.attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), P, B, H, N, d, out.data_ptr(),
                            lse.data_ptr(), _dtype_code(out), _stream(dev, stream))
    _check(st)
    return out, lse


def attn_bwd_workspace_bytes(B, H, N, d, dtype_code=ATTN_BF16):
    return int(library().attn_bwd_workspace_bytes(B, H, N, d, dtype_code))


def attn_bwd(q, k, v, o, do, lse, scale=None, *, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """dQ, dK, dV of sum(O * dO) (see attn_bwd in tiled_attn.h). bf16 tensors [B, H, N, d]."""
    import torch
    lib = library()
    _shape4("q", q)
    shape, dt, dev = tuple(q.shape), q.dtype, q.device
    for name, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _shape4(name, t, shape, dt, dev)
    B, H, N, d = shape
    _lse_out(lse, (B, H, N), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _shape4(name, t, shape, dt, dev)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    with _on_device(dev):
        st = lib.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                          lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                          workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          B, H, N, d, float(scale), code, _stream(dev, stream))
    _check(st)
    return dq, dk, dv


def attn_bwd_ex(q, k, v, o, do, lse, scale=None, *, causal=False, dq=None, dk=None, dv=None,
                workspace=None, stream=None):
    """dQ, dK, dV for q, o, do [B, H, Nq, d] and k, v [B, H, Nk, d] (see attn_bwd_ex). bf16."""
    import torch
    lib = library()
    _shape4("q", q)
    dt, dev = q.dtype, q.device
    B, H, Nq, d = q.shape
    _shape4("k", k, None, dt, dev)
    Nk = k.shape[2]
    _shape4("k", k, (B, H, Nk, d), dt, dev)
    _shape4("v", v, (B, H, Nk, d), dt, dev)
    for name, t in (("o", o), ("do", do)):
        _shape4(name, t, (B, H, Nq, d), dt, dev)
    _lse_out(lse, (B, H, Nq), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _shape4("dq", dq, (B, H, Nq, d), dt, dev)
    _shape4("dk", dk, (B, H, Nk, d), dt, dev)
    _shape4("dv", dv, (B, H, Nk, d), dt, dev)
    code = _dtype_code(q)
    need = attn_bwd_workspace_bytes(B, H, Nq, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    mask = ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE
    with _on_device(dev):
        st = lib.attn_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                             _ptr(dk), _ptr(dv), workspace.data_ptr(),
                             workspace.numel() * workspace.element_size(), B, H, Nq, Nk, d,
                             float(scale), mask, code, _stream(dev, stream))
    _check(st)
    return dq, dk, dv


def attn_bwd_ex_noalloc(q, k, v, o, do, lse, scale=None, *, causal=False, dq, dk, dv, stream=None):
    """attn_bwd_ex without a workspace (see attn_bwd_ex_noalloc in tiled_attn.h).

    The caller passes the outputs dq, dk, dv; the library allocates nothing.
    B * H * Nq must not exceed ATTN_NOALLOC_MAX_ROWS.
    """
    lib = library()
    _shape4("q", q)
    dt, dev = q.dtype, q.device
    B, H, Nq, d = q.shape
    _shape4("k", k, None, dt, dev)
    Nk = k.shape[2]
    _shape4("k", k, (B, H, Nk, d), dt, dev)
    _shape4("v", v, (B, H, Nk, d), dt, dev)
    for name, t in (("o", o), ("do", do), ("dq", dq)):
        _shape4(name, t, (B, H, Nq, d), dt, dev)
    _shape4("dk", dk, (B, H, Nk, d), dt, dev)
    _shape4("dv", dv, (B, H, Nk, d), dt, dev)
    _lse_out(lse, (B, H, Nq), dev)
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    mask = ATTN_MASK_CAUSAL if causal else ATTN_MASK_NONE
    import torch
    with _on_device(dev):
        st = lib.attn_bwd_ex_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                                     _ptr(dk), _ptr(dv), B, H, Nq, Nk, d, float(scale), mask,
                                     _dtype_code(q), _stream(dev, stream))
    _check(st)
    return dq, dk, dv


def attn_matmul_nt(a, b, *, out=None, stream=None):
    """C = A B^T for bf16 a [M, K] and b [N, K] (see attn_matmul_nt in tiled_attn.h)."""
    import torch
    lib = library()
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError(f"expected a [M, K] and b [N, K], got {tuple(a.shape)} and {tuple(b.shape)}")
    if a.dtype != b.dtype or a.device != b.device:
        raise ValueError("a and b must share dtype and device")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous")
    if a.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    M, K = a.shape
    N = b.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    if tuple(out.shape) != (M, N) or out.dtype != a.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor of the operands' dtype")
    with _on_device(a.device):
        st = lib.attn_matmul_nt(_ptr(a), _ptr(b), _ptr(out), M, N, K, _dtype_code(a),
                                _stream(a.device, stream))
    _check(st)
    return out


def attn_quantize_mxfp8(x, *, transpose=False, stream=None):
    """MXFP8 codes and scales (uint8 tensors) of bf16 x [..., rows, cols] (see attn_quantize_mxfp8).

    transpose=False: codes like x, scales [..., rows, cols/32]; transpose=True:
    codes [..., cols, rows], scales [..., cols, rows/32].
    """
    import torch
    lib = library()
    if x.dim() < 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous tensor [..., rows, cols]")
    if x.device.type != "cuda":
        raise ValueError("x must be on a GPU device")
    lead = tuple(x.shape[:-2])
    rows, cols = x.shape[-2], x.shape[-1]
    batch = 1
    for n in lead:
        batch *= n
    if transpose:
        q = torch.empty(lead + (cols, rows), dtype=torch.uint8, device=x.device)
        sc = torch.empty(lead + (cols, max(rows // 32, 0)), dtype=torch.uint8, device=x.device)
    else:
        q = torch.empty(lead + (rows, cols), dtype=torch.uint8, device=x.device)
        sc = torch.empty(lead + (rows, max(cols // 32, 0)), dtype=torch.uint8, device=x.device)
    with _on_device(x.device):
        st = lib.attn_quantize_mxfp8(_ptr(x), batch, rows, cols, 1 if transpose else 0, _ptr(q), _ptr(sc),
                                     _dtype_code(x), _stream(x.device, stream))
    _check(st)
    return q, sc


def _lse_out(lse, shape, device):
    """Checks a caller-supplied LSE output: a contiguous float32 tensor of `shape` on `device`."""
    import torch
    if tuple(lse.shape) != shape or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != device:
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {shape} on {device}")


def attn_fwd_mxfp8(q8, q_scales, k8, k_scales, vt8, vt_scales, scale=None, *, out=None, lse=None,
                   stream=None):
    """O (bf16), LSE of MXFP8 attention (see attn_fwd_mxfp8). q8, k8 [B,H,N,d]; vt8 [B,H,d,N]."""
    import torch
    lib = library()
    if q8.dim() != 4:
        raise ValueError(f"q8 must be [B, H, N, d], got {tuple(q8.shape)}")
    B, H, N, d = q8.shape
    shapes = {"q8": (q8, (B, H, N, d)), "q_scales": (q_scales, (B, H, N, d // 32)),
              "k8": (k8, (B, H, N, d)), "k_scales": (k_scales, (B, H, N, d // 32)),
              "vt8": (vt8, (B, H, d, N)), "vt_scales": (vt_scales, (B, H, d, N // 32))}
    for name, (t, shp) in shapes.items():
        if tuple(t.shape) != shp or t.dtype != torch.uint8 or not t.is_contiguous() or t.device != q8.device:
            raise ValueError(f"{name} must be a contiguous uint8 tensor of shape {shp} on {q8.device}")
    if out is not None:
        _shape4("out", out, (B, H, N, d), torch.bfloat16, q8.device)
    if lse is not None:
        _lse_out(lse, (B, H, N), q8.device)
    if q8.device.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    with _on_device(q8.device):
        st = lib.attn_fwd_mxfp8(_ptr(q8), _ptr(q_scales), _ptr(k8), _ptr(k_scales), _ptr(vt8), _ptr(vt_scales),
                                _ptr(out), _ptr(lse), B, H, N, d, float(scale), _stream(q8.device, stream))
    _check(st)
    return out, lse
