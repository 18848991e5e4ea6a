"""Pins for the oracle's integer block formats (CPU only).

INT4 and INT2 are two's complement codes with one UE8M0 scale per 32 K
elements (the integer tensor types of "Metal tensors でカスタム機械学習オペレーション
を最適化する", section "量子化データ型のネイティブサポート", with the block-wise
scale of its section "2-bit 量子化の限界圧縮を探る").  References that are not
the oracle: numpy's int8 sign extension for the value tables, a brute-force
nearest-integer search (ties to even) for the quantizer, exact rational
arithmetic for the GEMM, and closed forms (zero, scale bump).
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle

E4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _sext(codes, bits):
    """Two's complement value of `bits`-bit codes, by int8 sign extension."""
    c = np.asarray(codes, dtype=np.uint8)
    return ((c << (8 - bits)).astype(np.uint8).view(np.int8) >> (8 - bits)).astype(np.float64)


def test_int_tables():
    assert np.array_equal(oracle.int4_table(), _sext(np.arange(16), 4))
    assert np.array_equal(oracle.int2_table(), _sext(np.arange(4), 2))
    assert oracle.int4_table().min() == -8 and oracle.int4_table().max() == 7
    assert sorted(oracle.int2_table()) == [-2, -1, 0, 1]


def _unpack(q, elem, K):
    if elem == oracle.INT4:
        return _sext(np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], K), 4)
    return _sext(np.stack([(q >> (2 * i)) & 3 for i in range(4)], axis=-1).reshape(q.shape[0], K), 2)


LIMITS = {oracle.INT4: (-8, 7, 2), oracle.INT2: (-2, 1, 0)}   # qmin, qmax, emax


def _nearest_by_search(v, qmin, qmax):
    """The integer in [qmin, qmax] nearest to v (a Fraction), ties to the even
    one, by scanning every candidate."""
    best = None
    for q in range(qmin, qmax + 1):
        d = abs(v - q)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


def _ref_block(x, elem):
    qmin, qmax, emax = LIMITS[elem]
    if not np.isfinite(x).all():
        return 255, [0] * 32
    amax = max(abs(float(v)) for v in x)
    if amax == 0.0:
        e = -127
    else:
        e = math.frexp(amax)[1] - 1 - emax
        e = max(-127, min(127, e))
    vals = [_nearest_by_search(Fraction(float(v)) / Fraction(2) ** e, qmin, qmax) for v in x]
    return e + 127, vals


@pytest.mark.parametrize("elem", [oracle.INT4, oracle.INT2])
def test_int_quantizer_against_brute_force(elem):
    rng = np.random.default_rng(40 + elem)
    rows = 300
    x = (rng.standard_normal((rows, 64)) * np.exp2(rng.integers(-30, 30, size=(rows, 2))).repeat(32, 1)
         ).astype(np.float32)
    # ties on the integer grid of the block scale, exact saturation edges,
    # zeros, subnormals, a NaN and an infinity
    qmin, qmax, emax = LIMITS[elem]
    top = float(2 ** emax)
    x[0, :32] = np.float32(top)
    x[0, 1:32] = (np.arange(31) % (2 * (qmax - qmin) + 1) - (qmax - qmin)) / 2.0
    x[1, :32] = -np.float32(2 * top - 0.25)          # rounds to 2 top: saturates at qmin (reachable)
    x[1, 32:] = np.float32(2 * top - 0.25)           # saturates at qmax
    x[2] = 0.0
    x[3] = np.float32(1e-42)
    x[4, 3] = np.nan
    x[5, 40] = -np.inf
    q, s = oracle.quantize(x, elem)
    got = _unpack(q, elem, 64)
    for r in range(rows):
        for b in range(2):
            sb, vals = _ref_block(x[r, 32 * b:32 * b + 32], elem)
            assert s[r, b] == sb, (r, b)
            assert list(got[r, 32 * b:32 * b + 32]) == vals, (r, b)


@pytest.mark.parametrize("elem", [oracle.INT4, oracle.INT2])
def test_int_quantizer_invariants(elem):
    qmin, qmax, emax = LIMITS[elem]
    rng = np.random.default_rng(7 + elem)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    q, s = oracle.quantize(x, elem)
    v = _unpack(q, elem, 128)
    assert v.min() >= qmin and v.max() <= qmax
    # the block maximum lands in [2^emax, 2^(emax+1)) before rounding and
    # saturation, so every nonzero block uses a code of magnitude >= 2^emax
    blk = np.abs(v.reshape(200, 4, 32)).max(axis=2)
    assert (blk >= 2 ** emax).all()
    # dequantized values quantize back to themselves (same codes, same
    # scales), except in blocks holding the negative extreme code (-8 / -2):
    # its magnitude 2^(emax+1) selects the next scale up
    deq = (v.reshape(200, 4, 32) * np.exp2(s.astype(np.float64) - 127)[:, :, None]).reshape(200, 128)
    q2, s2 = oracle.quantize(deq.astype(np.float32), elem)
    v2 = _unpack(q2, elem, 128)
    extreme = (v.reshape(200, 4, 32) == qmin).any(axis=2)
    assert extreme.any() and (~extreme).any()
    assert np.array_equal(s2[~extreme], s[~extreme])
    assert np.array_equal(v2.reshape(200, 4, 32)[~extreme], v.reshape(200, 4, 32)[~extreme])
    assert np.array_equal(s2[extreme], s[extreme] + 1)


def _exact(aq, as_, ea, bq, bs, eb, M, N, K):
    def dec(q, e):
        if e == oracle.E4M3:
            return E4[q]
        return _unpack(q, e, K)

    A, B = dec(aq, ea), dec(bq, eb)
    C = np.zeros((M, N), dtype=object)
    for i in range(M):
        for j in range(N):
            c = Fraction(0)
            for k in range(K):
                sc = Fraction(2) ** (int(as_[i, k // 32]) - 127) * Fraction(2) ** (int(bs[j, k // 32]) - 127)
                c += Fraction(A[i, k]) * Fraction(B[j, k]) * sc
            C[i, j] = c
    return C


def _rand(rng, rows, K, elem):
    if elem == oracle.E4M3:
        q = rng.integers(0, 256, size=(rows, K), dtype=np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x7E
    else:
        q = rng.integers(0, 256, size=(rows, oracle.row_bytes(K, elem)), dtype=np.uint8)
    s = rng.integers(110, 140, size=(rows, K // 32), dtype=np.uint8)
    return q, s


@pytest.mark.parametrize("ea,eb,M,N,K", [(oracle.E4M3, oracle.INT4, 3, 4, 64), (oracle.E4M3, oracle.INT2, 4, 3, 96),
                                         (oracle.INT4, oracle.INT4, 2, 3, 32), (oracle.INT2, oracle.E4M3, 3, 2, 64)])
def test_int_gemm_exact_rationals(ea, eb, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + ea + eb)
    aq, as_ = _rand(rng, M, K, ea)
    bq, bs = _rand(rng, N, K, eb)
    C, ABS = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K)
    X = _exact(aq, as_, ea, bq, bs, eb, M, N, K)
    for i in range(M):
        for j in range(N):
            # block partials are exact in float64; only the cross-block sum rounds
            assert abs(Fraction(C[i, j]) - X[i, j]) <= Fraction(K // 32) * Fraction(2) ** -52 * Fraction(ABS[i, j])


def test_int_gemm_zero_and_scale_bump():
    rng = np.random.default_rng(3)
    M, N, K = 4, 5, 128
    aq, as_ = _rand(rng, M, K, oracle.E4M3)
    bq, bs = _rand(rng, N, K, oracle.INT4)
    C, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, np.zeros_like(bq), bs, oracle.INT4, M, N, K)
    assert (C == 0).all()
    base, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.INT4, M, N, K)
    bs2 = bs.copy()
    bs2[2, 1] += 1   # doubles block 1 of B row 2
    bumped, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs2, oracle.INT4, M, N, K)
    A = E4[aq] * np.exp2(as_.astype(np.float64) - 127).repeat(32, 1)
    Bv = _unpack(bq, oracle.INT4, K) * np.exp2(bs.astype(np.float64) - 127).repeat(32, 1)
    blk = (A[:, 32:64] * Bv[2, 32:64]).sum(axis=1)
    assert np.allclose(bumped[:, 2] - base[:, 2], blk, rtol=0, atol=1e-12 * np.abs(blk).max())
    others = [j for j in range(N) if j != 2]
    assert np.array_equal(bumped[:, others], base[:, others])


def test_int_gemm_gate_detects_flipped_code():
    rng = np.random.default_rng(5)
    M, N, K = 16, 16, 512
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    aq, as_ = oracle.quantize(a, oracle.E4M3)
    bq, bs = oracle.quantize(b, oracle.INT2)
    C, ABS = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.INT2, M, N, K)
    assert oracle.gate(C.astype(np.float32), C, ABS, K)["ok"]
    bq2 = bq.copy()
    bq2[5, 17] ^= 0x0C   # one INT2 code changes
    C2, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq2, bs, oracle.INT2, M, N, K)
    assert not oracle.gate(C2.astype(np.float32), C, ABS, K)["ok"]
