"""C-ABI checks that need no GPU: the library loads, exports every function
include/gvattn.h declares, and rejects every host-checkable problem with the
documented status before touching the device."""

import ctypes
import os
import re

import pytest

from segmented_varlen_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gvattn.h")

FAKE = 0x100000  # a non-null, 256-aligned pointer that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gvattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libgvattn.so not built")
    return B.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for need in ("gvattn_fwd", "gvattn_lse_merge", "gvattn_fwd_plan", "gvattn_fwd_run",
                 "gvattn_fwd_ranges", "gvattn_bwd", "gvattn_bwd_workspace_size",
                 "gvattn_fwd_workspace_size", "gvattn_status_string",
                 "gvattn_read_device_error", "gvattn_version", "gvattn_fwd_noalloc"):
        assert need in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"
        assert name in B.SIGNATURES, f"{name} has no binding signature"


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(GVATTN_[A-Z0-9_]+)\s+(\d+)", text))
    for k, v in consts.items():
        assert getattr(B, k) == int(v), k
    enums = dict(re.findall(r"(GVATTN_[A-Z0-9_]+)\s*=\s*(\d+)", text))
    for k, v in enums.items():
        assert getattr(B, k) == int(v), k


def test_version_and_status_strings(lib):
    assert lib.gvattn_version() == 100
    for rc in range(5):
        assert lib.gvattn_status_string(rc).startswith(b"GVATTN_")
    assert b"unknown" in lib.gvattn_status_string(99)


def test_workspace_size(lib):
    ws = lib.gvattn_fwd_workspace_size(64, 131072, 32, 8, 128, 128, B.GVATTN_BF16)
    assert ws > 256 and ws % 256 == 0
    # grows with the number of query rows, never depends on device data
    assert lib.gvattn_fwd_workspace_size(64, 2 * 131072, 32, 8, 128, 128, B.GVATTN_BF16) > ws
    assert lib.gvattn_fwd_workspace_size(64, 1000, 32, 7, 128, 128, B.GVATTN_BF16) == 0  # hq % hkv
    assert lib.gvattn_fwd_workspace_size(64, 1000, 32, 8, 96, 96, B.GVATTN_BF16) == 0   # head dim
    assert lib.gvattn_fwd_workspace_size(-1, 1000, 32, 8, 128, 128, B.GVATTN_BF16) == 0
    assert lib.gvattn_fwd_workspace_size(3, 192, 8, 2, 64, 64, B.GVATTN_FP32) > 0


def _fwd(lib, fn="gvattn_fwd", **over):
    args = dict(dtype=B.GVATTN_BF16, q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE,
                used_q=FAKE, used_k=FAKE, nseg=4, total_q=1024, total_k=1024, hq=8, hkv=2,
                d=128, dv=128, scale=0.125, causal=0, out=FAKE, lse=FAKE, ws=FAKE, ws_bytes=0,
                stream=None)
    args.update(over)
    return getattr(lib, fn)(*args.values())


@pytest.mark.parametrize("fn", ["gvattn_fwd", "gvattn_fwd_run"])
def test_fwd_host_validation(lib, fn):
    ok_ws = lib.gvattn_fwd_workspace_size(4, 1024, 8, 2, 128, 128, B.GVATTN_BF16)
    assert _fwd(lib, fn, dtype=5, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _fwd(lib, fn, d=96, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _fwd(lib, fn, dv=96, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _fwd(lib, fn, dv=0, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _fwd(lib, fn, hkv=3, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, hq=0, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, nseg=-1, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, total_q=-5, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, causal=2, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, scale=0.0, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, scale=-1.0, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, scale=float("inf"), ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd(lib, fn, scale=float("nan"), ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    for p in ("q", "k", "v", "cu_q", "cu_k", "used_q", "used_k", "out", "lse"):
        assert _fwd(lib, fn, ws_bytes=ok_ws, **{p: None}) == B.GVATTN_ERR_INVALID_ARG, p
    assert _fwd(lib, fn, ws=None, ws_bytes=ok_ws) == B.GVATTN_ERR_WORKSPACE
    assert _fwd(lib, fn, ws=FAKE + 8, ws_bytes=ok_ws) == B.GVATTN_ERR_WORKSPACE
    assert _fwd(lib, fn, ws_bytes=ok_ws - 1) == B.GVATTN_ERR_WORKSPACE
    # an empty launch is a no-op that needs nothing
    assert _fwd(lib, fn, nseg=0, q=None, ws=None) == B.GVATTN_OK


def test_noalloc_host_validation(lib):
    def call(**over):
        args = dict(dtype=B.GVATTN_BF16, q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, cu_k=FAKE,
                    used_q=FAKE, used_k=FAKE, nseg=4, total_q=1024, total_k=1024, hq=8, hkv=2,
                    d=128, dv=128, scale=0.125, causal=0, out=FAKE, lse=FAKE, stream=None)
        args.update(over)
        return lib.gvattn_fwd_noalloc(*args.values())
    assert call(dtype=5) == B.GVATTN_ERR_UNSUPPORTED
    assert call(d=96) == B.GVATTN_ERR_UNSUPPORTED
    assert call(hkv=3) == B.GVATTN_ERR_INVALID_ARG
    assert call(scale=float("nan")) == B.GVATTN_ERR_INVALID_ARG
    for p in ("q", "k", "v", "cu_q", "cu_k", "used_q", "used_k", "out", "lse"):
        assert call(**{p: None}) == B.GVATTN_ERR_INVALID_ARG, p
    # a plan larger than the static scratch is refused before any HIP call
    assert lib.gvattn_fwd_workspace_size(4, 1 << 30, 1, 1, 64, 64, B.GVATTN_BF16) > \
        B.GVATTN_NOALLOC_SCRATCH_BYTES
    assert call(total_q=1 << 30, hq=1, hkv=1, d=64, dv=64) == B.GVATTN_ERR_WORKSPACE
    assert call(nseg=0, q=None) == B.GVATTN_OK


def test_plan_host_validation(lib):
    ok_ws = lib.gvattn_fwd_workspace_size(4, 1024, 8, 2, 128, 64, B.GVATTN_BF16)  # d_v 64
    base = [B.GVATTN_BF16, FAKE, FAKE, FAKE, FAKE, 4, 1024, 1024, 8, 2, 128, 64, 1, FAKE, ok_ws,
            None]
    bad = list(base)
    bad[10] = 80
    assert lib.gvattn_fwd_plan(*bad) == B.GVATTN_ERR_UNSUPPORTED
    bad = list(base)
    bad[11] = 48
    assert lib.gvattn_fwd_plan(*bad) == B.GVATTN_ERR_UNSUPPORTED
    bad = list(base)
    bad[1] = None
    assert lib.gvattn_fwd_plan(*bad) == B.GVATTN_ERR_INVALID_ARG
    bad = list(base)
    bad[14] = 16
    assert lib.gvattn_fwd_plan(*bad) == B.GVATTN_ERR_WORKSPACE
    bad = list(base)
    bad[5] = 0
    assert lib.gvattn_fwd_plan(*bad) == B.GVATTN_OK


def _fwd_ranges(lib, **over):
    args = dict(dtype=B.GVATTN_BF16, q=FAKE, k=FAKE, v=FAKE, cu_q=FAKE, used_q=FAKE,
                kr_off=FAKE, kr_start=FAKE, kr_len=FAKE, nseg=4, nranges=9, total_q=1024,
                total_k=1024, hq=8, hkv=2, d=128, dv=256, scale=0.125, causal=0, out=FAKE,
                lse=FAKE, ws=FAKE, ws_bytes=0, stream=None)
    args.update(over)
    return lib.gvattn_fwd_ranges(*args.values())


def test_fwd_ranges_host_validation(lib):
    ok_ws = lib.gvattn_fwd_workspace_size(4, 1024, 8, 2, 128, 256, B.GVATTN_BF16)  # d_v 256
    assert _fwd_ranges(lib, dtype=5, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _fwd_ranges(lib, d=96, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _fwd_ranges(lib, hkv=3, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd_ranges(lib, nranges=-1, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd_ranges(lib, causal=3, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _fwd_ranges(lib, scale=0.0, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    for p in ("q", "k", "v", "cu_q", "used_q", "kr_off", "kr_start", "kr_len", "out", "lse"):
        assert _fwd_ranges(lib, ws_bytes=ok_ws, **{p: None}) == B.GVATTN_ERR_INVALID_ARG, p
    assert _fwd_ranges(lib, ws_bytes=ok_ws - 1) == B.GVATTN_ERR_WORKSPACE
    assert _fwd_ranges(lib, ws=FAKE + 16, ws_bytes=ok_ws) == B.GVATTN_ERR_WORKSPACE
    # no ranges at all needs no range arrays (validation only: nseg = 0)
    assert _fwd_ranges(lib, nseg=0, nranges=0, kr_start=None, kr_len=None) == B.GVATTN_OK


def _bwd(lib, **over):
    args = dict(dtype=B.GVATTN_BF16, q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE,
                cu_q=FAKE, cu_k=FAKE, used_q=FAKE, used_k=FAKE, nseg=4, total_q=1024,
                total_k=2048, hq=8, hkv=2, d=128, dv=64, scale=0.125, causal=1, dq=FAKE,
                dk=FAKE, dvv=FAKE, ws=FAKE, ws_bytes=0, stream=None)
    args.update(over)
    return lib.gvattn_bwd(*args.values())


def test_bwd_workspace_size(lib):
    n = lib.gvattn_bwd_workspace_size(4, 1024, 2048, 8, 2, 128, 64, B.GVATTN_BF16)
    assert n > 0 and n % 256 == 0
    # row statistics: 8 bytes per (query head, query row), so at least that
    assert n >= 8 * 8 * 1024
    assert lib.gvattn_bwd_workspace_size(4, 2048, 2048, 8, 2, 128, 64, B.GVATTN_BF16) > n
    assert lib.gvattn_bwd_workspace_size(4, 1024, 4096, 8, 2, 128, 64, B.GVATTN_BF16) > n
    assert lib.gvattn_bwd_workspace_size(4, 1024, 2048, 8, 2, 128, 64, B.GVATTN_FP16) == n
    # the backward is built for 16-bit types and head dims 64 / 128 only
    assert lib.gvattn_bwd_workspace_size(4, 1024, 2048, 8, 2, 128, 64, B.GVATTN_FP32) == 0
    assert lib.gvattn_bwd_workspace_size(4, 1024, 2048, 8, 2, 256, 64, B.GVATTN_BF16) == 0
    assert lib.gvattn_bwd_workspace_size(4, 1024, 2048, 8, 2, 128, 256, B.GVATTN_BF16) == 0
    assert lib.gvattn_bwd_workspace_size(4, 1024, 2048, 8, 3, 128, 64, B.GVATTN_BF16) == 0


def test_bwd_host_validation(lib):
    ok_ws = lib.gvattn_bwd_workspace_size(4, 1024, 2048, 8, 2, 128, 64, B.GVATTN_BF16)
    assert _bwd(lib, dtype=B.GVATTN_FP32, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _bwd(lib, dtype=7, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _bwd(lib, d=256, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _bwd(lib, dv=256, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _bwd(lib, d=96, ws_bytes=ok_ws) == B.GVATTN_ERR_UNSUPPORTED
    assert _bwd(lib, hkv=3, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _bwd(lib, causal=2, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _bwd(lib, scale=0.0, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _bwd(lib, scale=float("nan"), ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    assert _bwd(lib, total_k=-1, ws_bytes=ok_ws) == B.GVATTN_ERR_INVALID_ARG
    for p in ("q", "k", "v", "out", "dout", "lse", "cu_q", "cu_k", "used_q", "used_k", "dq",
              "dk", "dvv"):
        assert _bwd(lib, ws_bytes=ok_ws, **{p: None}) == B.GVATTN_ERR_INVALID_ARG, p
    assert _bwd(lib, ws=None, ws_bytes=ok_ws) == B.GVATTN_ERR_WORKSPACE
    assert _bwd(lib, ws=FAKE + 64, ws_bytes=ok_ws) == B.GVATTN_ERR_WORKSPACE
    assert _bwd(lib, ws_bytes=ok_ws - 1) == B.GVATTN_ERR_WORKSPACE
    assert _bwd(lib, nseg=0, q=None, ws=None) == B.GVATTN_OK


def test_merge_host_validation(lib):
    two = (ctypes.c_void_p * 2)(FAKE, FAKE)
    nine = (ctypes.c_void_p * 9)(*([FAKE] * 9))
    one_null = (ctypes.c_void_p * 2)(FAKE, None)
    p2 = ctypes.cast(two, ctypes.c_void_p)

    def merge(nparts=2, outs=p2, lses=p2, pd=B.GVATTN_BF16, od=B.GVATTN_BF16, nseg=4,
              total_q=100, hq=8, d=128, out=FAKE, lse=FAKE):
        return lib.gvattn_lse_merge(nparts, outs, lses, pd, od, FAKE, FAKE, nseg, total_q, hq, d,
                                    out, lse, None, None)

    assert merge(nparts=0) == B.GVATTN_ERR_INVALID_ARG
    assert merge(nparts=9, outs=ctypes.cast(nine, ctypes.c_void_p),
                 lses=ctypes.cast(nine, ctypes.c_void_p)) == B.GVATTN_ERR_UNSUPPORTED
    assert merge(pd=3) == B.GVATTN_ERR_UNSUPPORTED
    assert merge(d=100) == B.GVATTN_ERR_UNSUPPORTED
    assert merge(hq=0) == B.GVATTN_ERR_INVALID_ARG
    assert merge(out=None) == B.GVATTN_ERR_INVALID_ARG
    assert merge(outs=ctypes.cast(one_null, ctypes.c_void_p)) == B.GVATTN_ERR_INVALID_ARG
    assert merge(nseg=0) == B.GVATTN_OK
    assert merge(pd=B.GVATTN_FP16, od=B.GVATTN_FP32, nseg=0) == B.GVATTN_OK
    # out may be partial 0 only when both have one element type
    assert merge(pd=B.GVATTN_FP16, od=B.GVATTN_BF16) == B.GVATTN_ERR_INVALID_ARG
    assert merge(pd=B.GVATTN_FP32, od=B.GVATTN_FP16) == B.GVATTN_ERR_INVALID_ARG


def test_read_device_error_validation(lib):
    err = ctypes.c_int32(0)
    assert lib.gvattn_read_device_error(None, None, ctypes.byref(err)) == B.GVATTN_ERR_INVALID_ARG
    assert lib.gvattn_read_device_error(FAKE, None, None) == B.GVATTN_ERR_INVALID_ARG


def test_product_path_never_imports_the_oracle():
    """The package and its C++ sources do not reference the oracle."""
    pkg = os.path.join(ROOT, "segmented_varlen_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        B.load_library(str(tmp_path / "missing.so"))
