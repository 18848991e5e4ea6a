"""Pins for the oracle GEMMs and the tolerance gate (CPU only).

References that are not the oracle: exact rational arithmetic (fractions) over
values decoded by torch's float8 dtypes and the OCP E2M1 list, numpy float64
matmul where the scales are all 1, closed forms (identity, zero, scale bump),
and the accumulator-width example printed in the RIGEL summary.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden_kv, read_golden_rows

E4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
E5 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
E2 = np.array([float(v) for _, v in read_golden_rows("e2m1_values.txt")])


def _decode(q, elem, K):
    if elem == oracle.E4M3:
        return E4[q]
    if elem == oracle.E5M2:
        return E5[q]
    return E2[np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], K)]


def _rand_operand(rng, rows, K, elem, lo=110, hi=140, finite=True):
    if elem == oracle.E4M3:
        q = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        if finite:
            q[(q & 0x7F) == 0x7F] = 0x7E
    elif elem == oracle.E5M2:
        q = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        if finite:
            q[(q & 0x7C) == 0x7C] &= 0xFB   # exponent field 31 (inf / NaN) -> 30
    else:
        q = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    s = rng.integers(lo, hi, size=(rows, K // 32), dtype=np.uint8)
    return q, s


def _exact(aq, as_, ea, bq, bs, eb, M, N, K):
    """Exact rational C and sum|ab| from torch/OCP-decoded values."""
    A = _decode(aq, ea, K)
    B = _decode(bq, eb, K)
    C = [[Fraction(0)] * N for _ in range(M)]
    ABS = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            c = Fraction(0)
            a_ = Fraction(0)
            for k in range(K):
                sc = Fraction(2) ** (int(as_[i, k // 32]) - 127) * Fraction(2) ** (int(bs[j, k // 32]) - 127)
                p = Fraction(A[i, k]) * Fraction(B[j, k]) * sc
                c += p
                a_ += abs(p)
            C[i][j] = c
            ABS[i][j] = a_
    return C, ABS


@pytest.mark.parametrize("ea,eb,M,N,K,seed", [
    (oracle.E4M3, oracle.E4M3, 4, 4, 32, 1),
    (oracle.E4M3, oracle.E4M3, 3, 5, 96, 2),
    (oracle.E4M3, oracle.E2M1, 4, 4, 64, 3),
    (oracle.E2M1, oracle.E2M1, 2, 3, 64, 4),
    (oracle.E5M2, oracle.E5M2, 3, 4, 64, 5),
    (oracle.E4M3, oracle.E5M2, 4, 3, 32, 6),
    (oracle.E5M2, oracle.E4M3, 2, 4, 96, 7),
])
def test_bruteforce_exact_rationals(ea, eb, M, N, K, seed):
    rng = np.random.default_rng(seed)
    aq, as_ = _rand_operand(rng, M, K, ea)
    bq, bs = _rand_operand(rng, N, K, eb)
    C, ABS = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K)
    Cx, ABSx = _exact(aq, as_, ea, bq, bs, eb, M, N, K)
    nb = K // 32
    for i in range(M):
        for j in range(N):
            # only the cross-block float64 sum rounds: bound nb * 2^-53 * sum|ab|
            bound = Fraction(nb) * Fraction(1, 2 ** 53) * ABSx[i][j]
            assert abs(Fraction(C[i, j]) - Cx[i][j]) <= bound
            assert abs(Fraction(ABS[i, j]) - ABSx[i][j]) <= bound


def test_identity_gives_transposed_b():
    K = 64
    M = K
    N = 24
    rng = np.random.default_rng(5)
    aq = np.zeros((M, K), dtype=np.uint8)
    aq[np.arange(M), np.arange(K)] = 0x38          # 1.0
    as_ = np.full((M, K // 32), 127, dtype=np.uint8)
    bq, bs = _rand_operand(rng, N, K, oracle.E4M3)
    C, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    Bhat = _decode(bq, oracle.E4M3, K) * np.exp2(bs.astype(np.float64) - 127).repeat(32, axis=1)
    assert np.array_equal(C, Bhat.T)


def test_zero_operands():
    rng = np.random.default_rng(6)
    M, N, K = 8, 8, 64
    aq = np.zeros((M, K), dtype=np.uint8)
    as_ = rng.integers(0, 255, size=(M, K // 32), dtype=np.uint8)
    bq, bs = _rand_operand(rng, N, K, oracle.E4M3)
    C, ABS = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    assert (C == 0).all() and (ABS == 0).all()


def test_scale_bump_doubles_one_block():
    rng = np.random.default_rng(7)
    M, N, K = 6, 5, 128
    aq, as_ = _rand_operand(rng, M, K, oracle.E4M3)
    bq, bs = _rand_operand(rng, N, K, oracle.E4M3)
    C0, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    i, kb = 2, 1
    # contribution of block kb to row i: zero all other blocks of A
    aq_only = np.zeros_like(aq)
    aq_only[i, kb * 32:(kb + 1) * 32] = aq[i, kb * 32:(kb + 1) * 32]
    P, _ = oracle.mx_gemm(aq_only, as_, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    as2 = as_.copy()
    as2[i, kb] += 1
    C1, _ = oracle.mx_gemm(aq, as2, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    rows = [r for r in range(M) if r != i]
    assert np.array_equal(C1[rows], C0[rows])
    # exact up to the float64 cross-block rounding
    assert np.allclose(C1[i] - C0[i], P[i], rtol=0, atol=1e-12 * np.abs(P[i]).max() + 1e-300)
    assert np.array_equal(P[i] * 2, oracle.mx_gemm(aq_only, as2, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)[0][i])


def test_unit_scales_match_numpy_matmul():
    rng = np.random.default_rng(8)
    M, N, K = 33, 17, 256
    aq, _ = _rand_operand(rng, M, K, oracle.E4M3)
    bq, _ = _rand_operand(rng, N, K, oracle.E4M3)
    ones_a = np.full((M, K // 32), 127, dtype=np.uint8)
    ones_b = np.full((N, K // 32), 127, dtype=np.uint8)
    C, ABS = oracle.mx_gemm(aq, ones_a, oracle.E4M3, bq, ones_b, oracle.E4M3, M, N, K)
    A = _decode(aq, oracle.E4M3, K)
    B = _decode(bq, oracle.E4M3, K)
    ref = A @ B.T
    assert (np.abs(C - ref) <= 2 * K * 2.0 ** -53 * (np.abs(A) @ np.abs(B).T)).all()
    assert np.allclose(ABS, np.abs(A) @ np.abs(B).T, rtol=1e-15, atol=0)


def test_accumulator_width_example():
    g = read_golden_kv("accumulator_width.txt")
    K = int(g["K"])
    a = np.zeros((1, K), dtype=np.float32)
    a[0, 0] = g["terms_large"]
    a[0, 1:1 + int(g["count_small"])] = g["terms_small"]
    b = np.ones((1, K), dtype=np.float32)
    aq, as_ = oracle.quantize(a, oracle.E4M3)
    bq, bs = oracle.quantize(b, oracle.E4M3)
    # block 0 keeps 448 at scale 1; blocks 1..3 hold 2^-4 as 256 * 2^-12
    assert as_.tolist() == [[127, 115, 115, 115]]
    C, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, 1, 1, K)
    assert C[0, 0] == g["expected_total"]
    assert np.float32(C[0, 0]) == np.float32(g["expected_total"])
    # the page's fp16 stall value, reproduced with numpy half arithmetic
    acc = np.float16(g["terms_large"])
    for _ in range(int(g["count_small"])):
        acc = np.float16(acc + np.float16(g["terms_small"]))
    assert float(acc) == g["fp16_accumulator_total"]


def test_nan_scale_and_nan_code_propagate():
    rng = np.random.default_rng(9)
    M, N, K = 4, 4, 64
    aq, as_ = _rand_operand(rng, M, K, oracle.E4M3)
    bq, bs = _rand_operand(rng, N, K, oracle.E4M3)
    as_[1, 1] = 255
    bq[2, 5] = 0x7F
    C, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    assert np.isnan(C[1]).all()
    assert np.isnan(C[:, 2]).all()
    assert not np.isnan(C[np.ix_([0, 2, 3], [0, 1, 3])]).any()


def test_points_equal_full():
    rng = np.random.default_rng(10)
    M, N, K = 19, 23, 96
    for ea, eb in [(oracle.E4M3, oracle.E4M3), (oracle.E4M3, oracle.E2M1)]:
        aq, as_ = _rand_operand(rng, M, K, ea)
        bq, bs = _rand_operand(rng, N, K, eb)
        C, ABS = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K)
        I = rng.integers(0, M, 50)
        J = rng.integers(0, N, 50)
        Cp, ABSp = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K, points=(I, J))
        assert np.array_equal(Cp, C[I, J]) and np.array_equal(ABSp, ABS[I, J])


@pytest.mark.parametrize("b_is_nk", [0, 1])
def test_fp16_gemm_matches_numpy(b_is_nk):
    rng = np.random.default_rng(11)
    M, N, K = 21, 13, 200
    a = rng.uniform(-1, 1, (M, K)).astype(np.float16)
    b = rng.uniform(-1, 1, (K, N)).astype(np.float16)
    a[0, 0] = np.float16(6e-8)   # subnormal
    b_in = np.ascontiguousarray(b.T) if b_is_nk else b
    C, ABS = oracle.fp16_gemm(a.view(np.uint16), b_in.view(np.uint16), M, N, K, b_is_nk)
    A = a.astype(np.float64)
    B = b.astype(np.float64)
    assert (np.abs(C - A @ B) <= 2 * K * 2.0 ** -53 * (np.abs(A) @ np.abs(B))).all()
    I = np.array([0, 5, 20])
    J = np.array([0, 7, 12])
    Cp, _ = oracle.fp16_gemm(a.view(np.uint16), b_in.view(np.uint16), M, N, K, b_is_nk, points=(I, J))
    assert np.array_equal(Cp, C[I, J])


def test_gate_accepts_fp32_rounding_and_rejects_corruption():
    rng = np.random.default_rng(12)
    M, N, K = 16, 16, 256
    aq, as_ = _rand_operand(rng, M, K, oracle.E4M3)
    bq, bs = _rand_operand(rng, N, K, oracle.E4M3)
    C, ABS = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    # an fp32 sequential accumulation passes
    A = _decode(aq, oracle.E4M3, K) * np.exp2(as_.astype(np.float64) - 127).repeat(32, 1)
    B = _decode(bq, oracle.E4M3, K) * np.exp2(bs.astype(np.float64) - 127).repeat(32, 1)
    c32 = np.zeros((M, N), dtype=np.float32)
    for k in range(K):
        c32 = (c32 + (A[:, k:k + 1] * B[:, k][None, :]).astype(np.float32)).astype(np.float32)
    assert oracle.gate(c32, C, ABS, K)["ok"]
    # flipping one code byte of B changes some outputs beyond tolerance
    bq2 = bq.copy()
    bq2[3, 17] ^= 0x40
    C2, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq2, bs, oracle.E4M3, M, N, K)
    assert not oracle.gate(C2.astype(np.float32), C, ABS, K)["ok"]
    # bumping one scale byte of A as well
    as2 = as_.copy()
    as2[5, 2] += 1
    C3, _ = oracle.mx_gemm(aq, as2, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    assert not oracle.gate(C3.astype(np.float32), C, ABS, K)["ok"]
    # NaN where the reference is finite fails
    c_nan = C.astype(np.float32)
    c_nan[0, 0] = np.nan
    r = oracle.gate(c_nan, C, ABS, K)
    assert not r["ok"] and r["nan_mismatch"] == 1


def test_step_max_bruteforce():
    """The per-step magnitude the gate's matrix-unit term uses: for each
    output element, the sum over the 128-element steps of K of the largest
    |a_ik b_jk| * scales in the step, against a direct numpy evaluation over
    torch/OCP-decoded values (a ragged last step included)."""
    rng = np.random.default_rng(21)
    for ea, eb, M, N, K in ((oracle.E4M3, oracle.E4M3, 5, 7, 416), (oracle.E4M3, oracle.E2M1, 3, 4, 256),
                            (oracle.E5M2, oracle.E4M3, 4, 3, 96)):
        aq, as_ = _rand_operand(rng, M, K, ea, 100, 150)
        bq, bs = _rand_operand(rng, N, K, eb, 100, 150)
        C, ABS, SMAX = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K, step_max=True)
        A = _decode(aq, ea, K) * np.exp2(as_.astype(np.float64) - 127).repeat(32, 1)
        B = _decode(bq, eb, K) * np.exp2(bs.astype(np.float64) - 127).repeat(32, 1)
        P = np.abs(A[:, None, :] * B[None, :, :])          # M x N x K
        want = np.zeros((M, N))
        for k0 in range(0, K, 128):
            want += P[:, :, k0:k0 + 128].max(axis=2)
        assert np.array_equal(SMAX, want)
        C2, ABS2 = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K)
        assert np.array_equal(C, C2) and np.array_equal(ABS, ABS2)
        pts = (np.array([0, M - 1, 1]), np.array([N - 1, 0, 2]))
        _, _, SP = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K, points=pts, step_max=True)
        assert np.array_equal(SP, want[pts])


def test_gate_model_term_keeps_detection():
    """The matrix-unit term of the gate (kappa times the per-step largest
    product) still rejects a wrong scale byte and a flipped code on a
    realistic operand pair, and is what lets a single-step dominant-product
    error pass where the K-term bound alone does not."""
    from gpu_util import MFMA_STEP_KAPPA

    rng = np.random.default_rng(13)
    M, N, K = 32, 32, 1024
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    aq, as_ = oracle.quantize(a, oracle.E4M3)
    bq, bs = oracle.quantize(b, oracle.E4M3)
    C, ABS, SM = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K, step_max=True)
    kw = dict(step_max=SM, kappa=MFMA_STEP_KAPPA)
    assert oracle.gate(C.astype(np.float32), C, ABS, K, **kw)["ok"]
    as2 = as_.copy()
    as2[4, 9] += 1
    C2, _ = oracle.mx_gemm(aq, as2, oracle.E4M3, bq, bs, oracle.E4M3, M, N, K)
    assert not oracle.gate(C2.astype(np.float32), C, ABS, K, **kw)["ok"]
    bq2 = bq.copy()
    bq2[3, 100] ^= 0x40
    C3, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq2, bs, oracle.E4M3, M, N, K)
    assert not oracle.gate(C3.astype(np.float32), C, ABS, K, **kw)["ok"]
    # one step: 448 * 1 against 127 products of 2^-9; dropping the small ones
    # (an error of 127 * 2^-9 = 0.248) fails the K-term bound (128 * 2^-24 *
    # 448.25 = 0.0034) and passes with the model term when kappa * 448 covers it
    aq = np.full((1, 128), 0x01, dtype=np.uint8)
    aq[0, 0] = 0x7E
    bq = np.full((1, 128), 0x38, dtype=np.uint8)
    s1 = np.full((1, 4), 127, dtype=np.uint8)
    C, ABS, SM = oracle.mx_gemm(aq, s1, oracle.E4M3, bq, s1, oracle.E4M3, 1, 1, 128, step_max=True)
    assert C[0, 0] == 448 + 127 * 2.0 ** -9 and SM[0, 0] == 448
    dropped = np.array([[448.0]], dtype=np.float32)
    r = oracle.gate(dropped, C, ABS, 128)
    assert not r["ok"] and r["max_ratio"] > 50
    assert oracle.gate(dropped, C, ABS, 128, step_max=SM, kappa=2.0 ** -10)["ok"]
