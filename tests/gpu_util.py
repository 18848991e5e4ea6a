"""Helpers for the GPU parity tests: device setup, the HIP path through the
binding, and the oracle side on the same seeded inputs."""
import ctypes
import os
import sys

import numpy as np
import torch

import oracle
from block_scaled_precision_mxgemm_amd import inputs as mxin

DEV = "cuda:0"

FMT_ELEMS = {0: (oracle.E4M3, oracle.E4M3), 1: (oracle.E4M3, oracle.E2M1), 2: (oracle.E2M1, oracle.E2M1),
             3: (oracle.E5M2, oracle.E5M2), 4: (oracle.E4M3, oracle.E5M2), 5: (oracle.E5M2, oracle.E4M3),
             6: (oracle.E4M3, oracle.INT4), 7: (oracle.E4M3, oracle.INT2), 8: (oracle.E4M3, oracle.E2M3),
             9: (oracle.E4M3, oracle.E3M2)}

# Error model of one scaled-MFMA instruction (v_mfma_scale_f32_16x16x128_
# f8f6f4): the products of one 128-element step are added in one operation
# and bits far below the largest of them are dropped (measured: inside one
# 32-element block a product about 2^-14 below the block's largest is lost;
# across blocks of different scale products are kept to about 2^-27).
# tests/test_gpu_mfma_error.py measures single instructions on crafted,
# adversarial and random codes of every operand format and asserts
#   |instruction result - exact step sum| <= MFMA_STEP_KAPPA * max_k |a_k b_k|
#                                            + 2^-24 |exact step sum|;
# the largest measured ratio is 2^-8.6 (E4M3 x E4M3; E2M1 x E2M1 is exact to
# 2^-22), and the constant keeps a factor 3 of margin above it.
# Over K the error of a product is then at most the K-term accumulation bound
# plus MFMA_STEP_KAPPA times the sum over steps of each step's largest
# product (oracle.mx_gemm(..., step_max=True)).  Parity tests use the strict
# K-term bound unless they pass model=True; those cases are ones whose data
# put small products into a step beside a much larger one (few steps, or
# scales that vary block to block), where the strict bound cannot hold for
# this instruction.
MFMA_STEP_KAPPA = 2.0 ** -7


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def binding():
    from block_scaled_precision_mxgemm_amd import mxgemm

    return mxgemm


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def nan_canary(M, N):
    """Output buffer pre-filled with NaN: any element a kernel fails to write
    stays NaN and fails the NaN-position check of the gate."""
    return torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)


def gpu_quantize(x: np.ndarray, elem: int):
    b = binding()
    q, s = b.mxgemm_quantize(to_dev(x), elem)
    torch.cuda.synchronize()
    return q, s


_poison_lib = None


def poison_lds():
    """Fill every CU's LDS with 0xFF bytes (tests/hip/lds_poison.hip) on the
    current stream, so a kernel launched next that reads an LDS stage before
    its copy has landed sees NaN codes and scales (or -6 E2M1 nibbles), not
    bytes an earlier kernel happened to leave."""
    global _poison_lib
    if _poison_lib is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_build", "liblds_poison.so")
        if not os.path.exists(path):
            raise RuntimeError("test helper not built (run __graft_entry__.build()): " + path)
        lib = ctypes.CDLL(path)
        lib.lds_poison.argtypes = [ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p]
        lib.lds_poison.restype = ctypes.c_int
        _poison_lib = lib
    rc = _poison_lib.lds_poison(0xFFFFFFFF, 2048, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, "lds_poison launch failed: %d" % rc


def gpu_mx(a_q, a_s, b_q, b_s, fmt, M, N, dequant=False):
    b = binding()
    out = nan_canary(M, N)
    poison_lds()
    if dequant:
        b.mxgemm_run_dequant_fp16(a_q, a_s, b_q, b_s, fmt, out=out)
    else:
        b.mxgemm_run(a_q, a_s, b_q, b_s, fmt, out=out)
    torch.cuda.synchronize()
    return out


def mx_case(a32: np.ndarray, b32: np.ndarray, fmt: int, points=None, dequant=False, model=False):
    """Quantize both operands on the GPU and in the oracle (bytes must agree
    exactly), run the GPU GEMM on its own bytes and the oracle GEMM on the
    oracle's bytes; return (gate result, GPU C as numpy).  The gate is the
    strict K-term bound unless model=True (the scaled-MFMA step term is then
    added); 'max_ratio' is always the error over the strict bound."""
    ea, eb = FMT_ELEMS[fmt]
    M, K = a32.shape
    N = b32.shape[0]
    qa_o, sa_o = oracle.quantize(a32, ea)
    qb_o, sb_o = oracle.quantize(b32, eb)
    qa, sa = gpu_quantize(a32, ea)
    qb, sb = gpu_quantize(b32, eb)
    assert np.array_equal(qa.cpu().numpy(), qa_o), "A codes differ from the oracle quantizer"
    assert np.array_equal(sa.cpu().numpy(), sa_o), "A scales differ from the oracle quantizer"
    assert np.array_equal(qb.cpu().numpy(), qb_o), "B codes differ from the oracle quantizer"
    assert np.array_equal(sb.cpu().numpy(), sb_o), "B scales differ from the oracle quantizer"
    c = gpu_mx(qa, sa, qb, sb, fmt, M, N, dequant=dequant).cpu().numpy()
    ref, ab, sm = oracle.mx_gemm(qa_o, sa_o, ea, qb_o, sb_o, eb, M, N, K, points=points, step_max=True)
    got = c if points is None else c[points[0], points[1]]
    return model_gate(got, ref, ab, sm, K, model), c


def model_gate(got, ref, ab, sm, K, model):
    """oracle.gate with the scaled-MFMA step term when model is true; prints
    the error over the strict K-term bound and over the model bound either
    way."""
    strict = oracle.gate(got, ref, ab, K)
    with_model = oracle.gate(got, ref, ab, K, step_max=sm, kappa=MFMA_STEP_KAPPA)
    say("  max err / strict bound %.4g, / model bound %.4g%s" % (
        strict["max_ratio"], with_model["max_ratio_tol"], " (model gate applied)" if model else ""))
    return with_model if model else strict


def mx_sources(name, M=None, N=None, K=None, seed=None):
    return mxin.mx_sources(mxin.WORKLOADS[name], M, N, K, seed)
