"""Host-side checks of the C-ABI library (no GPU needed).

The library must load, export every function that include/w4a16.h declares,
and reject bad arguments before touching the device.  No call here passes
validation, so no kernel is ever launched.
"""

import ctypes

import pytest

import dequant_gemv_w4_amd as w4


def test_library_loads_and_exports_declared_symbols():
    L = w4.lib()
    declared = w4.declared_symbols()
    assert "w4_gemv" in declared and "w4_quantize" in declared and "w4_gemm" in declared
    for name in declared:
        assert hasattr(L, name), name


def test_format_version_and_status_strings():
    assert w4.w4_format_version() == 3
    assert w4.w4_status_string(0) == "ok"
    assert "gfx950" in w4.w4_status_string(6)
    assert w4.w4_status_string(99) == "unknown status"


def test_prepared_bytes_closed_form():
    # packed bytes rounded up to 256, then one 32-bit scale/zero word per group,
    # rows padded to a multiple of four
    assert w4.w4_prepared_bytes(8192, 8192) == 8192 * 4096 + 8192 * 64 * 4
    assert w4.w4_prepared_bytes(3, 384) == 768 + 4 * 3 * 4
    assert w4.w4_prepared_bytes(5, 128) == 512 + 8 * 1 * 4
    assert w4.w4_prepared_bytes(1, 100) == 0     # K not a multiple of 128
    assert w4.w4_prepared_bytes(0, 128) == 0
    # binary16 copy of X, then the rows' exponents and exactness flags (each 256-B aligned)
    assert w4.w4_gemm_workspace_bytes(4096, 28672, 8192) == 4096 * 8192 * 2 + 2 * 4096 * 4
    assert w4.w4_gemm_workspace_bytes(200, 300, 384) == 200 * 384 * 2 + 2 * 1024


def _fake(addr=0x100000):
    return ctypes.c_void_p(addr)


NULL = ctypes.c_void_p(None)


def test_validation_errors_before_device_work():
    L = w4.lib()
    s = NULL
    # null pointers
    assert L.w4_quantize(NULL, 0, 4, 128, _fake(), _fake(), _fake(), NULL, s) == 1
    assert L.w4_gemv(NULL, 4, 128, _fake(), 1, 1, _fake(), 0, s) == 1
    assert L.w4_gemm(_fake(), 4, 128, NULL, 1, _fake(), 0, NULL, 0, s) == 1
    assert L.w4_prepare(_fake(), NULL, _fake(), 4, 128, _fake(), 1 << 20, s) == 1
    # dtype
    assert L.w4_quantize(_fake(), 7, 4, 128, _fake(), _fake(), _fake(), NULL, s) == 4
    assert L.w4_gemv(_fake(), 4, 128, _fake(), 5, 1, _fake(), 0, s) == 4
    # shapes
    assert L.w4_quantize(_fake(), 0, 4, 100, _fake(), _fake(), _fake(), NULL, s) == 2
    assert L.w4_quantize(_fake(), 0, 0, 128, _fake(), _fake(), _fake(), NULL, s) == 2
    assert L.w4_gemv(_fake(), 4, 128, _fake(), 1, 0, _fake(), 0, s) == 2
    assert L.w4_gemv(_fake(), 4, 128, _fake(), 1, 17, _fake(), 0, s) == 2
    assert L.w4_gemv(_fake(), 4, 65536, _fake(), 1, 1, _fake(), 0, s) == 2
    assert L.w4_gemm(_fake(), 4, 192, _fake(), 4, _fake(), 0, NULL, 0, s) == 2
    # more output tiles than a grid holds
    big = 1 << 62
    assert L.w4_gemm(_fake(), 2**31 - 1, 128, _fake(), 65535 * 128, _fake(), 0, _fake(), big, s) == 2
    # K beyond W4_GEMM_MAX_K (2^20): the GEMM's 32-bit operand offsets
    assert L.w4_gemm(_fake(), 4, (1 << 20) + 128, _fake(), 4, _fake(), 0, _fake(), big, s) == 2
    assert L.w4_gemm_noalloc(_fake(), 4, (1 << 20) + 128, _fake(), 1, _fake(), 0, s) == 2
    assert w4.w4_gemm_workspace_bytes(4, 4, (1 << 20) + 128) == 0
    assert L.w4_fp8_gemm(_fake(), _fake(), 2**31 - 1, _fake(), _fake(), 2**31 - 1, 128, _fake(), 0, s) == 2
    assert L.w4_int8_gemm(_fake(), _fake(), 2**31 - 1, _fake(), _fake(), 2**31 - 1, 128, _fake(), 0, s) == 2
    # the fixed-workspace GEMM: validated like w4_gemm, and a workspace beyond its array
    # (M = 300 at K = 28672 needs 300 * 28672 * 2 bytes > 16 MiB) refused before device work
    assert L.w4_gemm_noalloc(_fake(), 4, 128, NULL, 1, _fake(), 0, s) == 1
    assert L.w4_gemm_noalloc(_fake(), 4, 128, _fake(), 1, _fake(), 3, s) == 4
    assert L.w4_gemm_noalloc(_fake(), 4, 192, _fake(), 4, _fake(), 0, s) == 2
    assert L.w4_gemm_noalloc(_fake(), 4, 128, _fake(), 0, _fake(), 0, s) == 2
    assert w4.w4_gemm_workspace_bytes(300, 4, 28672) > w4.GEMM_NOALLOC_MAX_WORKSPACE
    assert L.w4_gemm_noalloc(_fake(), 4, 28672, _fake(), 300, _fake(), 0, s) == 7
    assert w4.w4_gemm_workspace_bytes(256, 4, 28672) <= w4.GEMM_NOALLOC_MAX_WORKSPACE
    assert L.w4_gemm_noalloc(_fake(0x100010), 4, 28672, _fake(), 256, _fake(), 0, s) == 3
    # alignment
    assert L.w4_quantize(_fake(0x100004), 0, 4, 128, _fake(), _fake(), _fake(), NULL, s) == 3
    assert L.w4_gemv(_fake(0x100010), 4, 128, _fake(), 1, 1, _fake(), 0, s) == 3
    assert L.w4_gemv(_fake(), 4, 128, _fake(0x100008), 1, 1, _fake(), 0, s) == 3
    # destination too small
    assert L.w4_prepare(_fake(), _fake(), _fake(), 4, 128, _fake(), 10, s) == 9
    # the symmetric quantizer validates exactly as w4_quantize
    assert L.w4_quantize_symmetric(NULL, 0, 4, 128, _fake(), _fake(), _fake(), NULL, s) == 1
    assert L.w4_quantize_symmetric(_fake(), 7, 4, 128, _fake(), _fake(), _fake(), NULL, s) == 4
    assert L.w4_quantize_symmetric(_fake(), 0, 4, 100, _fake(), _fake(), _fake(), NULL, s) == 2
    assert L.w4_quantize_symmetric(_fake(0x100004), 0, 4, 128, _fake(), _fake(), _fake(), NULL, s) == 3


def test_python_layer_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        w4.w4_quantize(torch.zeros(4, 128))
    with pytest.raises(ValueError):
        w4.w4_quantize_symmetric(torch.zeros(4, 128))


def test_format_sizes_closed_form():
    F = w4.W4Format.make
    # group 32: K/32 scale/zero words per row, rows padded to four
    assert w4.w4_prepared_bytes_fmt(8192, 8192, F(32)) == 8192 * 4096 + 8192 * 256 * 4
    assert w4.w4_prepared_bytes_fmt(5, 256, F(64, True, 4)) == 768 + 8 * 4 * 4
    # group 128 with binary16 scales is the canonical layout, whatever the zeros
    assert w4.w4_prepared_bytes_fmt(3, 384, F(128, False, 4, True)) == w4.w4_prepared_bytes(3, 384)
    assert w4.w4_zeros_bytes(5, 256, F(32, True, 4)) == 20        # 40 groups, two per byte
    assert w4.w4_zeros_bytes(3, 128, F(128, False, 4)) == 2       # 3 groups -> 2 bytes
    assert w4.w4_zeros_bytes(3, 128, F(128)) == 3
    for bad in (F(16), F(256), F(128, False, 6), w4.W4Format(128, 2, 8, 0), w4.W4Format(128, 0, 8, 3)):
        assert w4.w4_zeros_bytes(4, 256, bad) == 0
        assert w4.w4_prepared_bytes_fmt(4, 256, bad) == 0
    assert w4.w4_prepared_bytes_fmt(4, 96, F(32)) == 0            # K must be a multiple of 128


def test_format_entry_points_validate_before_device_work():
    L = w4.lib()
    s = NULL
    ok = ctypes.byref(w4.W4Format.make(32, True, 4, False))
    bad = ctypes.byref(w4.W4Format.make(48))
    fnull = ctypes.POINTER(w4.W4Format)()
    # the format itself: missing, then outside the supported values
    assert L.w4_quantize_fmt(_fake(), 0, 4, 128, fnull, _fake(), _fake(), _fake(), NULL, s) == 1
    assert L.w4_quantize_fmt(_fake(), 0, 4, 128, bad, _fake(), _fake(), _fake(), NULL, s) == 5
    assert L.w4_prepare_fmt(_fake(), _fake(), _fake(), 4, 128, bad, _fake(), 1 << 20, s) == 5
    assert L.w4_unprepare_fmt(_fake(), 4, 128, bad, _fake(), _fake(), _fake(), s) == 5
    assert L.w4_gemv_fmt(_fake(), 4, 128, bad, _fake(), 1, 1, _fake(), 0, s) == 5
    # then the same checks as the canonical entry points
    assert L.w4_quantize_fmt(NULL, 0, 4, 128, ok, _fake(), _fake(), _fake(), NULL, s) == 1
    assert L.w4_quantize_fmt(_fake(), 7, 4, 128, ok, _fake(), _fake(), _fake(), NULL, s) == 4
    assert L.w4_quantize_fmt(_fake(), 0, 4, 96, ok, _fake(), _fake(), _fake(), NULL, s) == 2
    assert L.w4_quantize_fmt(_fake(0x100004), 0, 4, 128, ok, _fake(), _fake(), _fake(), NULL, s) == 3
    assert L.w4_prepare_fmt(_fake(), _fake(), _fake(), 4, 128, ok, _fake(), 10, s) == 9
    assert L.w4_gemv_fmt(_fake(), 4, 128, ok, _fake(), 1, 17, _fake(), 0, s) == 2
    assert L.w4_gemv_fmt(_fake(), 4, 128, ok, _fake(), 5, 1, _fake(), 0, s) == 4
    assert L.w4_gemv_fmt(_fake(0x100010), 4, 128, ok, _fake(), 1, 1, _fake(), 0, s) == 3
    # a canonical-layout format goes through w4_gemv's own checks
    canon = ctypes.byref(w4.W4Format.make(128, False, 4, True))
    assert L.w4_gemv_fmt(_fake(), 4, 128, canon, _fake(), 1, 0, _fake(), 0, s) == 2


def test_stream_read_validates_before_device_work():
    L = w4.lib()
    s = NULL
    assert L.w4_stream_read(NULL, 1024, _fake(), s) == 1
    assert L.w4_stream_read(_fake(), 1024, NULL, s) == 1
    assert L.w4_stream_read(_fake(), 0, _fake(), s) == 2
    assert L.w4_stream_read(_fake(), 1000, _fake(), s) == 2
    assert L.w4_stream_read(_fake(0x100008), 1024, _fake(), s) == 3
    assert L.w4_stream_read(_fake(), 1024, _fake(0x100002), s) == 3


def test_fp8_entry_points_validate_before_device_work():
    L = w4.lib()
    s = NULL
    f = _fake
    # null, dtype, shape (K a multiple of 128 within range, rows >= 1), alignment
    assert L.w4_fp8_quantize_rows(NULL, 0, 4, 128, f(), f(), NULL, s) == 1
    assert L.w4_fp8_quantize_rows(f(), 3, 4, 128, f(), f(), NULL, s) == 4
    assert L.w4_fp8_quantize_rows(f(), 0, 0, 128, f(), f(), NULL, s) == 2
    assert L.w4_fp8_quantize_rows(f(), 0, 4, 200, f(), f(), NULL, s) == 2
    assert L.w4_fp8_quantize_rows(f(), 0, 4, 1 << 17, f(), f(), NULL, s) == 2
    assert L.w4_fp8_quantize_rows(f(0x100008), 0, 4, 128, f(), f(), NULL, s) == 3
    assert L.w4_fp8_quantize_rows(f(), 1, 4, 128, f(0x100004), f(), NULL, s) == 3
    assert L.w4_fp8_gemm(f(), f(), 4, NULL, f(), 4, 128, f(), 0, s) == 1
    assert L.w4_fp8_gemm(f(), f(), 4, f(), f(), 4, 128, f(), 7, s) == 4
    assert L.w4_fp8_gemm(f(), f(), 0, f(), f(), 4, 128, f(), 0, s) == 2
    assert L.w4_fp8_gemm(f(), f(), 4, f(), f(), 4, 64, f(), 0, s) == 2
    assert L.w4_fp8_gemm(f(0x100004), f(), 4, f(), f(), 4, 128, f(), 0, s) == 3
    assert L.w4_fp8_gemm(f(), f(), 4, f(), f(), 4, 128, f(0x100002), 0, s) == 3


def test_int8_entry_points_validate_before_device_work():
    L = w4.lib()
    s = NULL
    f = _fake
    assert L.w4_int8_quantize_rows(NULL, 0, 4, 128, f(), f(), NULL, s) == 1
    assert L.w4_int8_quantize_rows(f(), 3, 4, 128, f(), f(), NULL, s) == 4
    assert L.w4_int8_quantize_rows(f(), 0, 4, 200, f(), f(), NULL, s) == 2
    assert L.w4_int8_quantize_rows(f(), 0, 4, 128, f(0x100008), f(), NULL, s) == 3
    assert L.w4_int8_gemm(f(), f(), 4, NULL, f(), 4, 128, f(), 0, s) == 1
    assert L.w4_int8_gemm(f(), f(), 4, f(), f(), 4, 128, f(), 7, s) == 4
    assert L.w4_int8_gemm(f(), f(), 4, f(), f(), 0, 128, f(), 0, s) == 2
    assert L.w4_int8_gemm(f(), f(), 4, f(), f(), 4, 128, f(0x100002), 0, s) == 3


def test_bench_refuses_more_than_one_gpu():
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert "error" in out and out["n_gpus"] == 2
