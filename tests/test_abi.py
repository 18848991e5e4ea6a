"""C-ABI checks that need no GPU: the library loads, exports every function
include/mxgemm.h declares, and rejects bad arguments before any launch (the
calls below return from argument validation; none reaches the device)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxgemm.h")
LIB = os.path.join(ROOT, "block_scaled_precision_mxgemm_amd", "libmxgemm.so")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mxgemm_\w+|fp16gemm_\w+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from block_scaled_precision_mxgemm_amd import build

        build.build_library()
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["mxgemm_quantize", "mxgemm_run", "fp16gemm_run", "mxgemm_run_dequant_fp16",
                                  "mxgemm_run_fused", "mxgemm_epilogue", "mxgemm_device_supported",
                                  "mxgemm_status_string", "mxgemm_mfma_ceiling"])


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def _run(lib, *args):
    f = lib.mxgemm_run
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p]
    return f(*args)


def test_validation_codes(lib):
    lib.mxgemm_status_string.restype = ctypes.c_char_p
    lib.mxgemm_status_string.argtypes = [ctypes.c_int]
    A = 0x1000
    ok = (A, A, A, A, A)
    assert _run(lib, None, A, A, A, A, 16, 16, 64, 0, None) == 1           # null pointer
    assert _run(lib, *ok, 16, 16, 48, 0, None) == 1                         # K % 32 != 0
    assert _run(lib, *ok, 0, 16, 64, 0, None) == 1                          # M = 0
    assert _run(lib, *ok, 16, -1, 64, 0, None) == 1                         # N < 0
    assert _run(lib, *ok, 16, 16, 64, 10, None) == 1                        # unknown fmt
    assert _run(lib, 0x1001, A, A, A, A, 16, 16, 64, 0, None) == 2          # misaligned A
    assert _run(lib, A, A, A, A, 0x1008, 16, 16, 64, 0, None) == 2          # misaligned C
    assert b"aligned" in lib.mxgemm_status_string(2)
    q = lib.mxgemm_quantize
    q.restype = ctypes.c_int
    q.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert q(A, 4, 64, 5, A, A, None) == 1                                  # unknown element
    assert q(A, 4, 40, 0, A, A, None) == 1                                  # K % 32 != 0
    assert q(0x1004, 4, 64, 0, A, A, None) == 2                             # misaligned X
    f = lib.fp16gemm_run
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p]
    assert f(A, A, A, 16, 16, 12, 0, None) == 1                             # K % 8 != 0
    assert f(A, A, A, 16, 16, 16, 2, None) == 1                             # bad layout flag
    d = lib.mxgemm_run_dequant_fp16
    d.restype = ctypes.c_int
    d.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p]
    assert d(*ok, 16, 16, 64, 1, None) == 1                                 # ablation is fp8 x fp8 only
    fu = lib.mxgemm_run_fused
    fu.restype = ctypes.c_int
    fu.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 3 + [ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                                                 ctypes.c_int, ctypes.c_void_p]
    assert fu(*ok, 16, 16, 64, 0, None, 2, 0, None) == 1                    # unknown activation
    assert fu(*ok, 16, 16, 64, 0, None, 0, 3, None) == 1                    # unknown output type
    assert fu(*ok, 16, 16, 64, 0, 0x1004, 1, 1, None) == 2                  # misaligned bias
    assert fu(A, A, A, A, 0x1008, 16, 16, 64, 0, None, 0, 1, None) == 2     # misaligned C
    assert fu(*ok, 16, 16, 48, 0, None, 0, 1, None) == 1                    # K % 32 != 0
    ep = lib.mxgemm_epilogue
    ep.restype = ctypes.c_int
    ep.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                   ctypes.c_void_p, ctypes.c_void_p]
    assert ep(None, 4, 4, None, 0, 0, A, None) == 1                         # null X
    assert ep(A, 0, 4, None, 0, 0, A, None) == 1                            # M = 0
    assert ep(A, 4, 4, None, 5, 0, A, None) == 1                            # unknown activation
    assert ep(A, 4, 4, None, 0, 9, A, None) == 1                            # unknown output type
    assert ep(A, 4, 4, 0x1002, 1, 1, A, None) == 2                          # misaligned bias
    assert ep(A, 4, 4, None, 0, 1, 0x1002, None) == 2                       # misaligned Y


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from block_scaled_precision_mxgemm_amd import mxgemm

    monkeypatch.setattr(mxgemm, "_lib", None)
    monkeypatch.setattr(mxgemm, "library_path", str(tmp_path / "missing.so"))
    with pytest.raises(mxgemm.MXGemmError):
        mxgemm.raw_library()


def test_ceiling_validation_codes(lib):
    f = lib.mxgemm_mfma_ceiling
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    A = 0x1000
    assert f(None, 4096, A, 64, 0, 10, 1, A, None, None) == 1        # null operands
    assert f(A, 16, A, 64, 0, 10, 1, A, None, None) == 1             # fewer than 32 operand bytes
    assert f(A, 4096, None, 0, 0, 10, 1, A, None, None) == 1         # MX kind without scales
    assert f(A, 4096, A, 64, 9, 10, 1, A, None, None) == 1           # unknown kind
    assert f(A, 4096, A, 64, 0, 0, 1, A, None, None) == 1            # no iterations
    assert f(A, 4096, A, 64, 0, 10, 0, A, None, None) == 1           # no workgroups
    assert f(0x1004, 4096, A, 64, 0, 10, 1, A, None, None) == 2      # misaligned operands
    assert f(A, 4096, 0x1001, 64, 0, 10, 1, A, None, None) == 2      # misaligned scales
    assert f(A, 4096, A, 64, 0, 10, 1, A, 0x1002, None) == 2         # misaligned clocks
