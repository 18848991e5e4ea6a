"""Helpers for the GPU parity tests: device setup, the HIP path through the
binding, and the oracle side on the same seeded inputs."""
import sys

import numpy as np
import torch

import oracle
from block_scaled_precision_mxgemm_amd import inputs as mxin

DEV = "cuda:0"

FMT_ELEMS = {0: (oracle.E4M3, oracle.E4M3), 1: (oracle.E4M3, oracle.E2M1), 2: (oracle.E2M1, oracle.E2M1),
             3: (oracle.E5M2, oracle.E5M2), 4: (oracle.E4M3, oracle.E5M2), 5: (oracle.E5M2, oracle.E4M3)}

# Per-dtype allowance of the scaled fp8/fp4 MFMA path, in units of
# 2^-24 * sum|a b|.  CDNA4's v_mfma_scale_f32_16x16x128_f8f6f4 does not add the
# up-to-128 products of one instruction exactly: measured on MI355X with
# single-instruction probes, it keeps roughly 16 significant bits relative to
# the largest product, giving up to ~600 units per instruction on the
# workloads' distributions (and ~5000 for adversarial random codes spanning
# the whole E4M3 range).  The K-term bound alone is met on every full-size
# workload (those tests pass extra_terms=0); small-K edge cases, where K units
# are fewer than one instruction's alignment error, get this allowance.
MFMA_ALIGNMENT_TERMS = 2048


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


def gpu_mx(a_q, a_s, b_q, b_s, fmt, M, N, dequant=False):
    b = binding()
    out = nan_canary(M, N)
    if dequant:
        b.mxgemm_run_dequant_fp16(a_q, a_s, b_q, b_s, fmt, out=out)
    else:
        b.mxgemm_run(a_q, a_s, b_q, b_s, fmt, out=out)
    torch.cuda.synchronize()
    return out


def mx_case(a32: np.ndarray, b32: np.ndarray, fmt: int, points=None, dequant=False, extra_terms=None):
    """Quantize both operands on the GPU and in the oracle (bytes must agree
    exactly), run the GPU GEMM on its own bytes and the oracle GEMM on the
    oracle's bytes; return (gate result, GPU C as numpy)."""
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
    if points is None:
        ref, ab = oracle.mx_gemm(qa_o, sa_o, ea, qb_o, sb_o, eb, M, N, K)
        got = c
    else:
        ref, ab = oracle.mx_gemm(qa_o, sa_o, ea, qb_o, sb_o, eb, M, N, K, points=points)
        got = c[points[0], points[1]]
    if extra_terms is None:
        extra_terms = 0 if dequant else MFMA_ALIGNMENT_TERMS
    return oracle.gate(got, ref, ab, K, extra_terms=extra_terms), c


def mx_sources(name, M=None, N=None, K=None, seed=None):
    return mxin.mx_sources(mxin.WORKLOADS[name], M, N, K, seed)
