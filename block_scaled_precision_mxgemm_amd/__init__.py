"""Block-scaled (MX) GEMM for AMD Instinct MI355X (gfx950).

The computation is C = (A * 2^sA)(B * 2^sB)^T over operands stored as FP8
(E4M3, E5M2), packed E2M1, packed FP6 (E2M3, E3M2) or packed INT4 / INT2 codes
with one UE8M0 scale per 32 contiguous K elements, fp32 output; a dense fp16
GEMM is the comparison path.  All arithmetic runs in the
HIP kernels of ``libmxgemm.so`` behind a C ABI (``include/mxgemm.h``); the
Python binding in :mod:`block_scaled_precision_mxgemm_amd.mxgemm` only
marshals torch device tensors to it.

Importing the package loads nothing; the binding is loaded on first use of one
of its names and raises if the HIP library has not been built.
"""
from __future__ import annotations

_BINDING_NAMES = (
    "mxgemm_quantize",
    "mxgemm_run",
    "mxgemm_run_fused",
    "mxgemm_epilogue",
    "fp16gemm_run",
    "mxgemm_run_dequant_fp16",
    "mxgemm_mfma_ceiling",
    "mxgemm_device_supported",
    "MXGemmError",
    "E4M3",
    "E5M2",
    "E2M1",
    "E2M3",
    "E3M2",
    "INT4",
    "INT2",
    "FMT_FP8_FP8",
    "FMT_FP8_FP4",
    "FMT_FP4_FP4",
    "FMT_BF8_BF8",
    "FMT_FP8_BF8",
    "FMT_BF8_FP8",
    "FMT_FP8_INT4",
    "FMT_FP8_INT2",
    "FMT_FP8_FP6",
    "FMT_FP8_BF6",
    "OUT_F32",
    "OUT_BF16",
    "OUT_F16",
    "ACT_NONE",
    "ACT_GELU",
    "CEIL_FP16",
    "library_path",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import mxgemm as _b

        return getattr(_b, name)
    raise AttributeError(name)
