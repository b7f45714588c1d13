"""Thin Python binding of the gvattn C ABI (include/gvattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libgvattn.so.  PyTorch supplies device memory and the current
stream.  The library is loaded on first use; if it has not been built the
call fails loudly (there is no fallback).
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libgvattn.so")

GVATTN_OK = 0
GVATTN_ERR_INVALID_ARG = 1
GVATTN_ERR_UNSUPPORTED = 2
GVATTN_ERR_WORKSPACE = 3
GVATTN_ERR_HIP = 4

GVATTN_FP32 = 0
GVATTN_BF16 = 1
GVATTN_FP16 = 2

GVATTN_DEVERR_USED_Q = 1
GVATTN_DEVERR_USED_K = 2
GVATTN_DEVERR_OFFSETS = 4
GVATTN_DEVERR_RANGE = 8
GVATTN_DEVERR_PLAN = 16
GVATTN_DEVERR_KRANGES = 32

GVATTN_MAX_PARTS = 8
GVATTN_WORKSPACE_ALIGN = 256
GVATTN_NOALLOC_SCRATCH_BYTES = 33554432

_lock = threading.Lock()
_lib = None

_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

_FWD_ARGS = [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
             _i32, _f32, _i32, _vp, _vp, _vp, _sz, _vp]

SIGNATURES = {
    "gvattn_fwd_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "gvattn_fwd": (ctypes.c_int, _FWD_ARGS),
    "gvattn_fwd_run": (ctypes.c_int, _FWD_ARGS),
    "gvattn_fwd_plan": (ctypes.c_int, [_i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _i32, _i32, _vp, _sz, _vp]),
    "gvattn_fwd_noalloc": (ctypes.c_int, [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                          _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp,
                                          _vp]),
    "gvattn_fwd_ranges": (ctypes.c_int, [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                         _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                         _vp, _vp, _vp, _sz, _vp]),
    "gvattn_lse_merge": (ctypes.c_int, [_i32, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32,
                                        _i32, _vp, _vp, _vp, _vp]),
    "gvattn_bwd_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "gvattn_bwd": (ctypes.c_int, [_i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                  _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp,
                                  _vp, _sz, _vp]),
    "gvattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gvattn_read_device_error": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(_i32)]),
    "gvattn_version": (ctypes.c_int, []),
}


def _bind_torch_runtime() -> None:
    """PyTorch ships its own HIP runtime (libamdhip64.so.7 in torch/lib).
    Importing torch before the library is opened makes the library bind to
    that runtime (same soname, already loaded) instead of loading the
    system copy next to it: two HIP runtimes in one process see the GPU
    inconsistently, and the second one to start can report no device."""
    try:
        import torch  # noqa: F401
    except ImportError:  # a process without torch uses the system runtime alone
        pass


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libgvattn.so (once) and declare the C signatures."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        _bind_torch_runtime()
        p = path or os.environ.get("GVATTN_LIBRARY") or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"libgvattn.so is not built ({p} missing); run "
                "`python -m segmented_varlen_attention_amd.build` first")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def status_string(rc: int) -> str:
    return load_library().gvattn_status_string(rc).decode()


def _check(rc: int, what: str) -> None:
    if rc != GVATTN_OK:
        raise RuntimeError(f"{what} failed: {status_string(rc)}")


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GVATTN_BF16
    if t.dtype == torch.float16:
        return GVATTN_FP16
    if t.dtype == torch.float32:
        return GVATTN_FP32
    raise ValueError(f"unsupported dtype {t.dtype}; expected bfloat16, float16 or float32")


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_i32_vec(t, n, name):
    torch = _torch()
    _need(t.dtype == torch.int32, f"{name} must be int32, got {t.dtype}")
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.dim() == 1 and t.shape[0] == n, f"{name} must have shape [{n}], got {tuple(t.shape)}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _fwd_common(q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse)):
        _need(t.is_cuda, f"{name} must be a device tensor")
        _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [rows, heads, dim]")
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    dv = v.shape[2]
    _need(tuple(v.shape[:2]) == (total_k, hkv),
          f"v must be {(total_k, hkv, 'd_v')}, got {tuple(v.shape)}")
    _need(dk == d, f"q and k head dims differ ({d} vs {dk})")
    _need(q.dtype == k.dtype == v.dtype == out.dtype, "q, k, v and out must share one dtype")
    _need(hq % hkv == 0, f"hq={hq} must be a multiple of hkv={hkv}")
    _need(tuple(out.shape) == (total_q, hq, dv),
          f"out must be {(total_q, hq, dv)}, got {tuple(out.shape)}")
    _need(lse.dtype == torch.float32 and tuple(lse.shape) == (hq, total_q),
          f"lse must be float32 [{hq}, {total_q}]")
    nseg = seqused_q.shape[0]
    _check_i32_vec(cu_seqlens_q, nseg + 1, "cu_seqlens_q")
    _check_i32_vec(cu_seqlens_k, nseg + 1, "cu_seqlens_k")
    _check_i32_vec(seqused_q, nseg, "seqused_q")
    _check_i32_vec(seqused_k, nseg, "seqused_k")
    return nseg, total_q, total_k, hq, hkv, d, dv


def gvattn_fwd_workspace_size(nseg: int, total_q: int, hq: int, hkv: int, d: int,
                              dtype: int, d_v: int | None = None) -> int:
    return int(load_library().gvattn_fwd_workspace_size(nseg, total_q, hq, hkv, d,
                                                        d if d_v is None else d_v, dtype))


def alloc_workspace(nseg: int, total_q: int, hq: int, hkv: int, d: int, dtype: int, device=None,
                    d_v: int | None = None):
    """Device workspace for gvattn_fwd (torch's allocator aligns to 512 B)."""
    torch = _torch()
    n = gvattn_fwd_workspace_size(nseg, total_q, hq, hkv, d, dtype, d_v)
    if n == 0:
        raise ValueError("invalid geometry for a workspace")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def _fwd_call(fn_name, q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse,
              softmax_scale, causal, workspace, stream):
    nseg, total_q, total_k, hq, hkv, d, dv = _fwd_common(
        q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse)
    dt = _dtype_code(q)
    if workspace is None:
        workspace = alloc_workspace(nseg, total_q, hq, hkv, d, dt, q.device, dv)
    lib = load_library()
    rc = getattr(lib, fn_name)(
        dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), seqused_q.data_ptr(), seqused_k.data_ptr(), nseg, total_q,
        total_k, hq, hkv, d, dv, float(softmax_scale), int(bool(causal)), out.data_ptr(),
        lse.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream_ptr(stream))
    _check(rc, fn_name)
    return workspace


def gvattn_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse,
               softmax_scale, causal=False, workspace=None, stream=None):
    """Segmented varlen attention forward into `out` / `lse` (used rows
    only).  Returns the workspace (reusable by gvattn_fwd_run)."""
    return _fwd_call("gvattn_fwd", q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k,
                     out, lse, softmax_scale, causal, workspace, stream)


def gvattn_fwd_run(q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse,
                   softmax_scale, causal, workspace, stream=None):
    """Forward on the plan already in `workspace` (from gvattn_fwd_plan or
    gvattn_fwd with the same geometry)."""
    _need(workspace is not None, "gvattn_fwd_run needs the planned workspace")
    return _fwd_call("gvattn_fwd_run", q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q,
                     seqused_k, out, lse, softmax_scale, causal, workspace, stream)


def gvattn_fwd_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse,
                       softmax_scale, causal=False, stream=None) -> None:
    """gvattn_fwd without a workspace: the library's static per-device
    scratch holds the plan (calls that overlap on one device race)."""
    nseg, total_q, total_k, hq, hkv, d, dv = _fwd_common(
        q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse)
    rc = load_library().gvattn_fwd_noalloc(
        _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
        cu_seqlens_k.data_ptr(), seqused_q.data_ptr(), seqused_k.data_ptr(), nseg, total_q,
        total_k, hq, hkv, d, dv, float(softmax_scale), int(bool(causal)), out.data_ptr(),
        lse.data_ptr(), _stream_ptr(stream))
    _check(rc, "gvattn_fwd_noalloc")


def gvattn_fwd_ranges(q, k, v, cu_seqlens_q, seqused_q, kr_off, kr_start, kr_len, out, lse,
                      softmax_scale, causal=False, workspace=None, stream=None):
    """Forward where segment s's keys are the K/V row ranges
    [kr_start[i], kr_start[i] + kr_len[i]), i in [kr_off[s], kr_off[s+1]),
    concatenated in order.  Returns the workspace."""
    nseg = seqused_q.shape[0]
    # reuse the shape checks of the prefix form with stand-in key vectors
    _, total_q, total_k, hq, hkv, d, dv = _fwd_common(
        q, k, v, cu_seqlens_q, cu_seqlens_q, seqused_q, seqused_q, out, lse)
    _check_i32_vec(kr_off, nseg + 1, "kr_off")
    nranges = kr_start.shape[0] if kr_start.dim() == 1 else -1
    _check_i32_vec(kr_start, nranges, "kr_start")
    _check_i32_vec(kr_len, nranges, "kr_len")
    dt = _dtype_code(q)
    if workspace is None:
        workspace = alloc_workspace(nseg, total_q, hq, hkv, d, dt, q.device, dv)
    rc = load_library().gvattn_fwd_ranges(
        dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
        seqused_q.data_ptr(), kr_off.data_ptr(),
        kr_start.data_ptr() if nranges > 0 else None,
        kr_len.data_ptr() if nranges > 0 else None, nseg, nranges, total_q, total_k, hq, hkv,
        d, dv, float(softmax_scale), int(bool(causal)), out.data_ptr(), lse.data_ptr(),
        workspace.data_ptr(), workspace.numel(), _stream_ptr(stream))
    _check(rc, "gvattn_fwd_ranges")
    return workspace


def gvattn_bwd_workspace_size(nseg: int, total_q: int, total_k: int, hq: int, hkv: int, d: int,
                              d_v: int, dtype: int) -> int:
    return int(load_library().gvattn_bwd_workspace_size(nseg, total_q, total_k, hq, hkv, d, d_v,
                                                        dtype))


def gvattn_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k,
               dq, dk, dv, softmax_scale, causal=False, workspace=None, stream=None):
    """Gradients of gvattn_fwd: writes dq, dk, dv for the used rows and keys
    (other rows untouched).  `out` / `lse` are the forward's outputs for the
    same inputs, `dout` the gradient of `out`.  Returns the workspace."""
    torch = _torch()
    nseg, total_q, total_k, hq, hkv, d, d_v = _fwd_common(
        q, k, v, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, out, lse)
    for name, t, ref in (("dout", dout, out), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _need(t.is_cuda and t.is_contiguous(), f"{name} must be a contiguous device tensor")
        _need(t.dtype == ref.dtype and tuple(t.shape) == tuple(ref.shape),
              f"{name} must be {ref.dtype} {tuple(ref.shape)}, got {t.dtype} {tuple(t.shape)}")
    dt = _dtype_code(q)
    if workspace is None:
        n = gvattn_bwd_workspace_size(nseg, total_q, total_k, hq, hkv, d, d_v, dt)
        if n == 0:
            raise ValueError("gvattn_bwd: unsupported dtype or head dim, or invalid geometry")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    rc = load_library().gvattn_bwd(
        dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
        lse.data_ptr(), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), seqused_q.data_ptr(),
        seqused_k.data_ptr(), nseg, total_q, total_k, hq, hkv, d, d_v, float(softmax_scale),
        int(bool(causal)), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
        workspace.numel(), _stream_ptr(stream))
    _check(rc, "gvattn_bwd")
    return workspace


def gvattn_fwd_plan(dtype: int, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, total_q: int,
                    total_k: int, hq: int, hkv: int, d: int, causal: bool, workspace=None,
                    stream=None, d_v: int | None = None):
    """Build the tile plan of a geometry into `workspace` (allocated when
    None) and return the workspace."""
    nseg = seqused_q.shape[0]
    _check_i32_vec(cu_seqlens_q, nseg + 1, "cu_seqlens_q")
    _check_i32_vec(cu_seqlens_k, nseg + 1, "cu_seqlens_k")
    _check_i32_vec(seqused_q, nseg, "seqused_q")
    _check_i32_vec(seqused_k, nseg, "seqused_k")
    if workspace is None:
        workspace = alloc_workspace(nseg, total_q, hq, hkv, d, dtype, seqused_q.device, d_v)
    rc = load_library().gvattn_fwd_plan(
        dtype, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), seqused_q.data_ptr(),
        seqused_k.data_ptr(), nseg, total_q, total_k, hq, hkv, d, d if d_v is None else d_v,
        int(bool(causal)),
        workspace.data_ptr(), workspace.numel(), _stream_ptr(stream))
    _check(rc, "gvattn_fwd_plan")
    return workspace


def gvattn_lse_merge(part_outs, part_lses, cu_seqlens_q, seqused_q, out, lse,
                     device_error=None, stream=None) -> None:
    """FP32 LSE merge of partial (O_p, LSE_p) results into `out` / `lse`
    (used rows only; `out`/`lse` may be part_outs[0]/part_lses[0])."""
    torch = _torch()
    n = len(part_outs)
    _need(n == len(part_lses) and n >= 1, "need as many partial LSEs as outputs (>= 1)")
    _need(n <= GVATTN_MAX_PARTS, f"at most {GVATTN_MAX_PARTS} partitions")
    total_q, hq, d = out.shape
    for po, pl in zip(part_outs, part_lses):
        _need(po.is_cuda and po.is_contiguous() and tuple(po.shape) == (total_q, hq, d),
              f"partial outputs must be contiguous device [{total_q}, {hq}, {d}]")
        _need(po.dtype == part_outs[0].dtype, "partial outputs must share one dtype")
        _need(pl.is_cuda and pl.is_contiguous() and pl.dtype == torch.float32
              and tuple(pl.shape) == (hq, total_q), f"partial LSEs must be float32 [{hq}, {total_q}]")
    _need(out.is_cuda and out.is_contiguous(), "out must be a contiguous device tensor")
    _need(lse.is_cuda and lse.is_contiguous() and lse.dtype == torch.float32
          and tuple(lse.shape) == (hq, total_q), f"lse must be float32 [{hq}, {total_q}]")
    nseg = seqused_q.shape[0]
    _check_i32_vec(cu_seqlens_q, nseg + 1, "cu_seqlens_q")
    _check_i32_vec(seqused_q, nseg, "seqused_q")
    outs = (ctypes.c_void_p * n)(*[p.data_ptr() for p in part_outs])
    lses = (ctypes.c_void_p * n)(*[p.data_ptr() for p in part_lses])
    err_ptr = 0
    if device_error is not None:
        _need(device_error.dtype == torch.int32 and device_error.is_cuda, "device_error must be a device int32")
        err_ptr = device_error.data_ptr()
    rc = load_library().gvattn_lse_merge(
        n, ctypes.cast(outs, ctypes.c_void_p), ctypes.cast(lses, ctypes.c_void_p),
        _dtype_code(part_outs[0]), _dtype_code(out), cu_seqlens_q.data_ptr(),
        seqused_q.data_ptr(), nseg, total_q, hq, d, out.data_ptr(), lse.data_ptr(),
        err_ptr or None, _stream_ptr(stream))
    _check(rc, "gvattn_lse_merge")


def gvattn_read_device_error(workspace, stream=None) -> int:
    """Synchronises and returns the workspace's GVATTN_DEVERR_* bits."""
    err = _i32(0)
    rc = load_library().gvattn_read_device_error(workspace.data_ptr(), _stream_ptr(stream),
                                                 ctypes.byref(err))
    _check(rc, "gvattn_read_device_error")
    return int(err.value)


def gvattn_version() -> int:
    return int(load_library().gvattn_version())
