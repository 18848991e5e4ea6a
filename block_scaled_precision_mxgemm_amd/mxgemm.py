"""Python binding of libmxgemm.so (C ABI in include/mxgemm.h).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked, outputs are allocated with torch when not given, and the device
pointers plus the current HIP stream are handed to the library.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.  If
the library has not been built, loading fails with MXGemmError.
"""
from __future__ import annotations

import ctypes
import os

import torch

E4M3 = 0
E5M2 = 1
E2M3 = 2
E3M2 = 3
E2M1 = 4
INT4 = 8
INT2 = 9
FMT_FP8_FP8 = 0
FMT_FP8_FP4 = 1
FMT_FP4_FP4 = 2
FMT_BF8_BF8 = 3
FMT_FP8_BF8 = 4
FMT_BF8_FP8 = 5
FMT_FP8_INT4 = 6
FMT_FP8_INT2 = 7
FMT_FP8_FP6 = 8
FMT_FP8_BF6 = 9

_FMT_ELEMS = {FMT_FP8_FP8: (E4M3, E4M3), FMT_FP8_FP4: (E4M3, E2M1), FMT_FP4_FP4: (E2M1, E2M1),
              FMT_BF8_BF8: (E5M2, E5M2), FMT_FP8_BF8: (E4M3, E5M2), FMT_BF8_FP8: (E5M2, E4M3),
              FMT_FP8_INT4: (E4M3, INT4), FMT_FP8_INT2: (E4M3, INT2), FMT_FP8_FP6: (E4M3, E2M3),
              FMT_FP8_BF6: (E4M3, E3M2)}

# output types and activations of the fused epilogue (MXG_OUT_*, MXG_ACT_*)
OUT_F32 = 0
OUT_BF16 = 1
OUT_F16 = 2
ACT_NONE = 0
ACT_GELU = 1
# kind of mxgemm_mfma_ceiling beside the FMT_* pairs
CEIL_FP16 = 16
_OUT_DTYPES = {OUT_F32: torch.float32, OUT_BF16: torch.bfloat16, OUT_F16: torch.float16}

library_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxgemm.so")


class MXGemmError(RuntimeError):
    pass


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise MXGemmError("libmxgemm.so is not built (run __graft_entry__.build() or "
                          "python -m block_scaled_precision_mxgemm_amd.build): " + library_path)
    lib = ctypes.CDLL(library_path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.mxgemm_quantize.argtypes = [p, i64, i64, ci, p, p, p]
    lib.mxgemm_quantize.restype = ci
    lib.mxgemm_run.argtypes = [p, p, p, p, p, i64, i64, i64, ci, p]
    lib.mxgemm_run.restype = ci
    lib.mxgemm_run_dequant_fp16.argtypes = [p, p, p, p, p, i64, i64, i64, ci, p]
    lib.mxgemm_run_dequant_fp16.restype = ci
    lib.mxgemm_run_fused.argtypes = [p, p, p, p, p, i64, i64, i64, ci, p, ci, ci, p]
    lib.mxgemm_run_fused.restype = ci
    lib.mxgemm_epilogue.argtypes = [p, i64, i64, p, ci, ci, p, p]
    lib.mxgemm_epilogue.restype = ci
    lib.fp16gemm_run.argtypes = [p, p, p, i64, i64, i64, ci, p]
    lib.fp16gemm_run.restype = ci
    lib.mxgemm_mfma_ceiling.argtypes = [p, i64, p, i64, ci, i64, ci, p, p, p]
    lib.mxgemm_mfma_ceiling.restype = ci
    lib.mxgemm_device_supported.argtypes = []
    lib.mxgemm_device_supported.restype = ci
    lib.mxgemm_status_string.argtypes = [ci]
    lib.mxgemm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = _load().mxgemm_status_string(rc).decode()
        raise MXGemmError("%s failed: status %d (%s)" % (what, rc, msg))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_u8(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(name + " must be a GPU tensor")
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e5m2, torch.float8_e8m0fnu):
        t = t.view(torch.uint8)
    if t.dtype != torch.uint8:
        raise TypeError(name + " must hold uint8 codes")
    if not t.is_contiguous():
        raise ValueError(name + " must be contiguous")
    return t


def _row_bytes(K: int, elem: int) -> int:
    if elem in (E2M1, INT4):
        return K // 2
    if elem == INT2:
        return K // 4
    if elem in (E2M3, E3M2):
        return K // 4 * 3
    return K


def mxgemm_device_supported() -> bool:
    rc = _load().mxgemm_device_supported()
    if rc < 0:
        _check(-rc, "mxgemm_device_supported")
    return rc == 1


def mxgemm_quantize(x: torch.Tensor, elem: int = E4M3, q: torch.Tensor | None = None,
                    s: torch.Tensor | None = None, stream=None):
    """Quantize fp32 rows (rows x K, K contiguous) to (codes, scales), uint8 tensors."""
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float32 GPU tensor")
    rows, K = x.shape
    if q is None:
        q = torch.empty((rows, _row_bytes(K, elem)), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    q = _dev_u8(q, "q")
    s = _dev_u8(s, "s")
    if q.shape != (rows, _row_bytes(K, elem)) or s.shape != (rows, K // 32):
        raise ValueError("output shapes do not match x")
    rc = _load().mxgemm_quantize(x.data_ptr(), rows, K, elem, q.data_ptr(), s.data_ptr(), _stream(stream))
    _check(rc, "mxgemm_quantize")
    return q, s


def _mx_args(a_q, a_s, b_q, b_s, fmt, out, out_dtype=torch.float32):
    if fmt not in _FMT_ELEMS:
        raise ValueError("unknown fmt %r" % (fmt,))
    ea, eb = _FMT_ELEMS[fmt]
    a_q = _dev_u8(a_q, "a_q")
    a_s = _dev_u8(a_s, "a_s")
    b_q = _dev_u8(b_q, "b_q")
    b_s = _dev_u8(b_s, "b_s")
    M, nb = a_s.shape
    N = b_s.shape[0]
    K = nb * 32
    if a_q.shape != (M, _row_bytes(K, ea)) or b_q.shape != (N, _row_bytes(K, eb)) or b_s.shape != (N, nb):
        raise ValueError("operand shapes disagree: A %s/%s, B %s/%s" %
                         (tuple(a_q.shape), tuple(a_s.shape), tuple(b_q.shape), tuple(b_s.shape)))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_q.device)
    if out.dtype != out_dtype or out.shape != (M, N) or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous M x N %s GPU tensor" % (out_dtype,))
    return a_q, a_s, b_q, b_s, out, M, N, K


def _bias_arg(bias, N):
    if bias is None:
        return None
    if bias.dtype != torch.float32 or not bias.is_cuda or bias.shape != (N,) or not bias.is_contiguous():
        raise ValueError("bias must be a contiguous float32 GPU tensor of N values")
    return bias


def mxgemm_run(a_q, a_s, b_q, b_s, fmt: int = FMT_FP8_FP8, out: torch.Tensor | None = None, stream=None):
    """C = (A * 2^sA)(B * 2^sB)^T in fp32; A: M x K codes, B: N x K codes."""
    a_q, a_s, b_q, b_s, out, M, N, K = _mx_args(a_q, a_s, b_q, b_s, fmt, out)
    rc = _load().mxgemm_run(a_q.data_ptr(), a_s.data_ptr(), b_q.data_ptr(), b_s.data_ptr(), out.data_ptr(),
                            M, N, K, fmt, _stream(stream))
    _check(rc, "mxgemm_run")
    return out


def mxgemm_run_fused(a_q, a_s, b_q, b_s, fmt: int = FMT_FP8_FP8, bias: torch.Tensor | None = None,
                     act: int = ACT_NONE, out_type: int = OUT_F32, out: torch.Tensor | None = None, stream=None):
    """mxgemm_run with the output step fused into the GEMM: C = out_type(act(A B^T + bias)).
    bias: N float32 values or None; act: ACT_NONE / ACT_GELU; out_type: OUT_F32 /
    OUT_BF16 / OUT_F16 (the output tensor's dtype float32 / bfloat16 / float16)."""
    if out_type not in _OUT_DTYPES:
        raise ValueError("unknown out_type %r" % (out_type,))
    a_q, a_s, b_q, b_s, out, M, N, K = _mx_args(a_q, a_s, b_q, b_s, fmt, out, _OUT_DTYPES[out_type])
    bias = _bias_arg(bias, N)
    rc = _load().mxgemm_run_fused(a_q.data_ptr(), a_s.data_ptr(), b_q.data_ptr(), b_s.data_ptr(), out.data_ptr(),
                                  M, N, K, fmt, None if bias is None else bias.data_ptr(), act, out_type,
                                  _stream(stream))
    _check(rc, "mxgemm_run_fused")
    return out


def mxgemm_epilogue(x: torch.Tensor, bias: torch.Tensor | None = None, act: int = ACT_NONE,
                    out_type: int = OUT_F32, out: torch.Tensor | None = None, stream=None):
    """The same output step as a separate pass over an fp32 M x N matrix x."""
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float32 GPU tensor")
    if out_type not in _OUT_DTYPES:
        raise ValueError("unknown out_type %r" % (out_type,))
    M, N = x.shape
    if out is None:
        out = torch.empty((M, N), dtype=_OUT_DTYPES[out_type], device=x.device)
    if out.dtype != _OUT_DTYPES[out_type] or out.shape != (M, N) or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("out must be a contiguous M x N %s GPU tensor" % (_OUT_DTYPES[out_type],))
    bias = _bias_arg(bias, N)
    rc = _load().mxgemm_epilogue(x.data_ptr(), M, N, None if bias is None else bias.data_ptr(), act, out_type,
                                 out.data_ptr(), _stream(stream))
    _check(rc, "mxgemm_epilogue")
    return out


def mxgemm_run_dequant_fp16(a_q, a_s, b_q, b_s, fmt: int = FMT_FP8_FP8, out: torch.Tensor | None = None,
                            stream=None):
    """Ablation: dequantize to fp16 in registers, then fp16 MFMA (fp8 x fp8 only)."""
    a_q, a_s, b_q, b_s, out, M, N, K = _mx_args(a_q, a_s, b_q, b_s, fmt, out)
    rc = _load().mxgemm_run_dequant_fp16(a_q.data_ptr(), a_s.data_ptr(), b_q.data_ptr(), b_s.data_ptr(),
                                         out.data_ptr(), M, N, K, fmt, _stream(stream))
    _check(rc, "mxgemm_run_dequant_fp16")
    return out


def fp16gemm_run(a: torch.Tensor, b: torch.Tensor, b_is_nk: bool, out: torch.Tensor | None = None, stream=None):
    """fp16 GEMM with fp32 output. a: M x K; b: N x K if b_is_nk else K x N."""
    for name, t in (("a", a), ("b", b)):
        if t.dtype not in (torch.float16, torch.int16, torch.uint16) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(name + " must be a contiguous fp16 GPU tensor")
    M, K = a.shape
    N = b.shape[0] if b_is_nk else b.shape[1]
    if (b.shape[1] if b_is_nk else b.shape[0]) != K:
        raise ValueError("inner dimensions disagree")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=a.device)
    if out.dtype != torch.float32 or out.shape != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous M x N float32 tensor")
    rc = _load().fp16gemm_run(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K, 1 if b_is_nk else 0,
                              _stream(stream))
    _check(rc, "fp16gemm_run")
    return out


def mxgemm_mfma_ceiling(ops: torch.Tensor, scales: torch.Tensor | None, kind: int, iters: int, workgroups: int,
                        out: torch.Tensor | None = None, clocks: torch.Tensor | None = None, stream=None):
    """Measurement helper: run `iters` rounds of the large GEMM's 32-MFMA
    compute phase per wave on fragments taken from the bytes of `ops` (and
    scale registers from `scales`), `workgroups` workgroups of 8 waves, no
    memory traffic.  kind: an FMT_* pair or CEIL_FP16.  Returns `out`
    (workgroups * 512 floats).  Flops: workgroups * 8 * iters * 32 * 65536
    (CEIL_FP16: workgroups * 8 * iters * 64 * 16384).  clocks (optional,
    workgroups * 2 int32): shader cycles and 100 MHz ticks of each
    workgroup's first wave over its MFMA loop."""
    if not ops.is_cuda or not ops.is_contiguous():
        raise ValueError("ops must be a contiguous GPU tensor")
    if scales is not None and (not scales.is_cuda or not scales.is_contiguous()):
        raise ValueError("scales must be a contiguous GPU tensor")
    if out is None:
        out = torch.empty(workgroups * 512, dtype=torch.float32, device=ops.device)
    if out.dtype != torch.float32 or out.numel() < workgroups * 512 or not out.is_contiguous():
        raise ValueError("out must hold workgroups * 512 contiguous floats")
    if clocks is not None and (clocks.dtype != torch.int32 or clocks.numel() < 2 * workgroups
                               or not clocks.is_contiguous()):
        raise ValueError("clocks must hold workgroups * 2 contiguous int32")
    rc = _load().mxgemm_mfma_ceiling(ops.data_ptr(), ops.numel() * ops.element_size(),
                                     None if scales is None else scales.data_ptr(),
                                     0 if scales is None else scales.numel() * scales.element_size(),
                                     kind, iters, workgroups, out.data_ptr(),
                                     None if clocks is None else clocks.data_ptr(), _stream(stream))
    _check(rc, "mxgemm_mfma_ceiling")
    return out


def raw_library():
    """The loaded ctypes library (for ABI-level tests)."""
    return _load()
