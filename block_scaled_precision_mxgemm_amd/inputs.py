"""Seeded synthetic inputs for the MX GEMM workloads.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no quantization, no decoding, no products).  Both the CPU
oracle's tests and the GPU path take their fp32 / fp16 sources from here, so
the two sides see identical inputs.

Generator: numpy ``default_rng(seed)`` (PCG64), float32 draws, A drawn before B.
B is always drawn directly in the layout the path consumes (N x K for the MX
operands).  Recipes per workload:

  mxfp8_256     256^3,  A, B ~ N(0, 1)
  fp16_1024     1024^3, A (M x K), B (K x N row-major) ~ U(-1, 1), rounded to fp16
  mxfp8_2048    2048^3, A, B ~ N(0, 1) * 2^u with one u ~ U{-6..6} per
                (row, 32-element K block), drawn independently for A and B
  prefill       M=8192 x N=14336 x K=4096; A ~ N(0, 1) with each element
                multiplied by 50 with probability 0.001; B ~ N(0, 0.02) (std);
                the MXFP4 x MXFP4 prefill takes the same sources
  decode        M=16 x N=28672 x K=8192; A ~ N(0, 1) (MXFP8), B ~ N(0, 0.02)
                (MXFP4, E2M1 codes)
  mxfp8_8192    8192^3, A, B ~ N(0, 1); the E4M3 x E5M2 8192^3 product takes
                the same sources
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    seed: int
    elem_a: str  # "e4m3" | "e5m2" | "e2m1" | "e2m3" | "e3m2" | "int4" | "int2" | "fp16"
    elem_b: str
    recipe: str
    description: str


WORKLOADS = {
    w.name: w
    for w in [
        Workload("mxfp8_256", 256, 256, 256, 1, "e4m3", "e4m3", "normal",
                 "MXFP8 GEMM 256^3, N(0,1) operands"),
        Workload("fp16_1024", 1024, 1024, 1024, 2, "fp16", "fp16", "uniform_fp16",
                 "dense fp16 GEMM 1024^3, U(-1,1), row-major A and B"),
        Workload("mxfp8_2048", 2048, 2048, 2048, 3, "e4m3", "e4m3", "normal_blockpow2",
                 "MXFP8 GEMM 2048^3, N(0,1) x 2^U{-6..6} per 32-K block"),
        Workload("prefill_8192x14336x4096", 8192, 14336, 4096, 4, "e4m3", "e4m3", "prefill",
                 "LLM-prefill MXFP8 GEMM, 8192 tokens x 4096 -> 14336"),
        Workload("prefill_mxfp4_8192x14336x4096", 8192, 14336, 4096, 4, "e2m1", "e2m1", "prefill",
                 "LLM-prefill MXFP4 x MXFP4 GEMM (both operands E2M1), same sources"),
        Workload("prefill_e2m3_8192x14336x4096", 8192, 14336, 4096, 4, "e4m3", "e2m3", "prefill",
                 "LLM-prefill GEMM, MXFP8 activations x FP6 E2M3 weights, same sources"),
        Workload("prefill_int4_8192x14336x4096", 8192, 14336, 4096, 4, "e4m3", "int4", "prefill",
                 "LLM-prefill GEMM, MXFP8 activations x INT4 weights (UE8M0 per 32), same sources"),
        Workload("prefill_int2_8192x14336x4096", 8192, 14336, 4096, 4, "e4m3", "int2", "prefill",
                 "LLM-prefill GEMM, MXFP8 activations x INT2 weights (UE8M0 per 32), same sources"),
        Workload("decode_16x28672x8192", 16, 28672, 8192, 5, "e4m3", "e2m1", "decode",
                 "decode MXFP8 x MXFP4 GEMM, 16 tokens x 8192 -> 28672"),
        Workload("mxfp8_8192", 8192, 8192, 8192, 6, "e4m3", "e4m3", "normal",
                 "MXFP8 GEMM 8192^3, N(0,1) operands"),
        Workload("mxfp8xbf8_8192", 8192, 8192, 8192, 6, "e4m3", "e5m2", "normal",
                 "MX GEMM 8192^3, E4M3 A x E5M2 B, the same N(0,1) sources"),
        Workload("decode_int4_16x28672x8192", 16, 28672, 8192, 5, "e4m3", "int4", "decode",
                 "decode GEMM, MXFP8 activations x INT4 weights (UE8M0 per 32), the decode sources"),
        Workload("decode_int2_16x28672x8192", 16, 28672, 8192, 5, "e4m3", "int2", "decode",
                 "decode GEMM, MXFP8 activations x INT2 weights (UE8M0 per 32), the decode sources"),
        Workload("decode_e2m3_16x28672x8192", 16, 28672, 8192, 5, "e4m3", "e2m3", "decode",
                 "decode GEMM, MXFP8 activations x FP6 E2M3 weights (UE8M0 per 32), the decode sources"),
        Workload("decode_e3m2_16x28672x8192", 16, 28672, 8192, 5, "e4m3", "e3m2", "decode",
                 "decode GEMM, MXFP8 activations x FP6 E3M2 weights (UE8M0 per 32), the decode sources"),
    ]
}


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _blockpow2(rng, shape):
    rows, K = shape
    z = rng.standard_normal(shape, dtype=np.float32)
    u = rng.integers(-6, 7, size=(rows, K // 32))  # inclusive -6..6
    mult = np.exp2(u.astype(np.float32))
    return (z.reshape(rows, K // 32, 32) * mult[:, :, None]).reshape(rows, K)


def mx_sources(w: Workload, M: int | None = None, N: int | None = None,
               K: int | None = None, seed: int | None = None):
    """fp32 sources (A: M x K, B: N x K) for an MX workload.

    M/N/K/seed override the workload's sizes (same recipe), for small parity
    cases of the same distribution.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    rng = np.random.default_rng(w.seed if seed is None else seed)
    if w.recipe == "normal":
        a = _normal(rng, (M, K))
        b = _normal(rng, (N, K))
    elif w.recipe == "normal_blockpow2":
        a = _blockpow2(rng, (M, K))
        b = _blockpow2(rng, (N, K))
    elif w.recipe == "prefill":
        a = _normal(rng, (M, K))
        outl = rng.random((M, K), dtype=np.float32) < np.float32(0.001)
        a[outl] *= np.float32(50.0)
        b = _normal(rng, (N, K), 0.02)
    elif w.recipe == "decode":
        a = _normal(rng, (M, K))
        b = _normal(rng, (N, K), 0.02)
    else:
        raise ValueError("not an MX workload: " + w.name)
    return a, b


def decode_weight_copies(w: Workload, copies: int, N: int | None = None, K: int | None = None):
    """Independent fp32 weight sets for the decode workload (seeds seed*1000+c),
    used to rotate weights so that repeated launches stream them from HBM.
    A generator: one set is held in host memory at a time."""
    N = w.N if N is None else N
    K = w.K if K is None else K
    for c in range(copies):
        rng = np.random.default_rng(w.seed * 1000 + c)
        yield _normal(rng, (N, K), 0.02)


def fp16_sources(w: Workload, b_is_nk: bool, M: int | None = None, N: int | None = None,
                 K: int | None = None, seed: int | None = None):
    """fp16 operands (numpy float16): A is M x K; B is K x N, or N x K if b_is_nk.

    For the dense fp16 workload the entries are U(-1, 1) rounded to fp16 (RNE).
    For an MX workload the fp16 pair uses the same fp32 sources the MX run
    quantizes, rounded to fp16 (the paired comparison run).
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    if w.recipe == "uniform_fp16":
        rng = np.random.default_rng(w.seed if seed is None else seed)
        a = rng.uniform(-1.0, 1.0, size=(M, K)).astype(np.float32).astype(np.float16)
        b = rng.uniform(-1.0, 1.0, size=(K, N)).astype(np.float32).astype(np.float16)
        if b_is_nk:
            b = np.ascontiguousarray(b.T)
        return a, b
    a, b = mx_sources(w, M, N, K, seed)  # b is N x K
    a16 = a.astype(np.float16)
    b16 = b.astype(np.float16)
    if not b_is_nk:
        b16 = np.ascontiguousarray(b16.T)
    return a16, b16


def sample_points(M: int, N: int, count: int, seed: int = 12345, tile: int = 256):
    """Output coordinates for sampled parity: every tile's four corners and
    centre (so each workgroup tile and the ragged tail are hit), the global
    last row/column, then uniform random points up to ``count``."""
    rng = np.random.default_rng(seed)
    pts = set()
    for i0 in range(0, M, tile):
        for j0 in range(0, N, tile):
            i1 = min(i0 + tile, M) - 1
            j1 = min(j0 + tile, N) - 1
            for i, j in ((i0, j0), (i0, j1), (i1, j0), (i1, j1), ((i0 + i1) // 2, (j0 + j1) // 2)):
                pts.add((i, j))
    pts.add((M - 1, N - 1))
    extra = max(0, count - len(pts))
    I = rng.integers(0, M, size=extra)
    J = rng.integers(0, N, size=extra)
    for i, j in zip(I.tolist(), J.tolist()):
        pts.add((i, j))
    arr = np.array(sorted(pts), dtype=np.int64)
    return arr[:, 0].copy(), arr[:, 1].copy()
