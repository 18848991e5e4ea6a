"""Pins for the oracle's FP6 element formats (CPU only).

E2M3 and E3M2 follow the OCP Microscaling definitions (the pages name FP6
only as an operand type of the scaled matrix unit, beside E5M2, and give no
bit layout): E2M3 = sign, 2 exponent bits (bias 1), 3 mantissa bits; E3M2 =
sign, 3 exponent bits (bias 3), 2 mantissa bits; no NaN, no infinity; one
UE8M0 scale per 32 K elements; 6-bit codes packed little-endian (element k at
bits 6k .. 6k+5 of the row).  References that are not the oracle: torch's
float8_e4m3fn and float8_e5m2 dtypes (every FP6 value must be one of theirs,
exactly), the formats' closed forms (largest value, smallest subnormal,
strict monotonicity of the codes), numpy's little-endian bit unpacking, a
brute-force nearest search with ties to the even code, and exact rational
arithmetic for the GEMM.
"""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle

FP6 = {oracle.E2M3: dict(ebits=2, mbits=3, bias=1, vmax=7.5, sub=0.125, emax=2),
       oracle.E3M2: dict(ebits=3, mbits=2, bias=3, vmax=28.0, sub=0.0625, emax=4)}


def _table(elem):
    return oracle.e2m3_table() if elem == oracle.E2M3 else oracle.e3m2_table()


@pytest.mark.parametrize("elem", [oracle.E2M3, oracle.E3M2])
def test_fp6_values_are_fp8_values(elem):
    """Every FP6 value is exactly an E4M3 and an E5M2 (E3M2) value: a
    round trip through torch's fp8 dtypes leaves it unchanged."""
    t = _table(elem)
    x = torch.tensor(t, dtype=torch.float64)
    assert torch.equal(x.to(torch.float8_e4m3fn).to(torch.float64), x)
    if elem == oracle.E3M2:
        assert torch.equal(x.to(torch.float8_e5m2).to(torch.float64), x)
    else:
        # 3 mantissa bits: some E2M3 values are not E5M2 values
        assert not torch.equal(x.to(torch.float8_e5m2).to(torch.float64), x)


@pytest.mark.parametrize("elem", [oracle.E2M3, oracle.E3M2])
def test_fp6_closed_forms(elem):
    f = FP6[elem]
    t = _table(elem)
    pos, neg = t[:32], t[32:]
    assert np.array_equal(neg, -pos) and pos[0] == 0.0 and math.copysign(1.0, neg[0]) == -1.0
    # strictly increasing magnitudes over the 32 codes of one sign
    assert (np.diff(pos) > 0).all()
    assert pos.max() == f["vmax"] and pos[1] == f["sub"]
    # the largest is (2 - 2^-mbits) * 2^((2^ebits - 1) - bias); the smallest
    # normal is 2^(1 - bias), at code 2^mbits
    assert f["vmax"] == (2 - 2.0 ** -f["mbits"]) * 2.0 ** ((2 ** f["ebits"] - 1) - f["bias"])
    assert pos[2 ** f["mbits"]] == 2.0 ** (1 - f["bias"])
    # subnormal codes are evenly spaced, one subnormal step apart
    assert np.array_equal(pos[:2 ** f["mbits"]], np.arange(2 ** f["mbits"]) * f["sub"])
    # emax: the exponent of the largest power of two not above the largest value
    assert 2.0 ** f["emax"] <= f["vmax"] < 2.0 ** (f["emax"] + 1)


def _unpack6(q, K):
    """6-bit codes of packed rows (little-endian bit order), independently of the oracle."""
    bits = np.unpackbits(q, axis=1, bitorder="little")[:, : 6 * K].reshape(q.shape[0], K, 6)
    return (bits * (1 << np.arange(6))).sum(axis=2).astype(np.int64)


def _nearest_code(v, t):
    """Code of the nearest value of table t (32 magnitudes) to |v| (a
    Fraction), ties to the code with the even last bit; saturated."""
    a = abs(v)
    best = None
    for c in range(32):
        d = abs(a - Fraction(t[c]))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    code = best[1]
    return code | (32 if v < 0 else 0)


def _ref_block(x, elem):
    f = FP6[elem]
    t = _table(elem)
    if not np.isfinite(x).all():
        return 255, [0] * 32
    amax = max(abs(float(v)) for v in x)
    if amax == 0.0:
        e = -127
    else:
        e = max(-127, min(127, math.frexp(amax)[1] - 1 - f["emax"]))
    codes = []
    for v in x:
        fv = Fraction(float(v)) / Fraction(2) ** e
        c = _nearest_code(fv, t)
        if fv == 0 and math.copysign(1.0, float(v)) < 0:
            c = 32
        codes.append(c)
    return e + 127, codes


@pytest.mark.parametrize("elem", [oracle.E2M3, oracle.E3M2])
def test_fp6_quantizer_against_brute_force(elem):
    f = FP6[elem]
    t = _table(elem)
    rng = np.random.default_rng(60 + elem)
    rows = 200
    x = (rng.standard_normal((rows, 64)) * np.exp2(rng.integers(-30, 30, size=(rows, 2))).repeat(32, 1)
         ).astype(np.float32)
    # exact midpoints between adjacent representable values (ties), the
    # block maximum pinned to 2^emax so the scale is 2^0
    top = 2.0 ** f["emax"]
    mids = [(t[c] + t[c + 1]) / 2 for c in range(31)]
    x[0, 0] = top
    x[0, 1:32] = np.array(mids, dtype=np.float32)
    x[1, 0] = top
    x[1, 1:32] = -np.array(mids, dtype=np.float32)
    x[2, :32] = np.float32(2 * top - 2.0 ** -20)    # rounds past the largest value: saturates
    x[3] = 0.0
    x[4, 5] = np.nan
    x[5, 33] = np.inf
    x[6, :32] = np.float32(1e-40)
    q, s = oracle.quantize(x, elem)
    got = _unpack6(q, 64)
    for r in range(rows):
        for b in range(2):
            sb, codes = _ref_block(x[r, 32 * b:32 * b + 32], elem)
            assert s[r, b] == sb, (r, b)
            assert list(got[r, 32 * b:32 * b + 32]) == codes, (r, b)


def _exact(aq, as_, ea, bq, bs, eb, M, N, K):
    def dec(q, e):
        if e == oracle.E4M3:
            return torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return _table(e)[_unpack6(q, K)]

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
        q = rng.integers(0, 256, size=(rows, K // 4 * 3), dtype=np.uint8)
    s = rng.integers(110, 140, size=(rows, K // 32), dtype=np.uint8)
    return q, s


@pytest.mark.parametrize("ea,eb,M,N,K", [(oracle.E4M3, oracle.E2M3, 3, 4, 64), (oracle.E4M3, oracle.E3M2, 4, 3, 96),
                                         (oracle.E2M3, oracle.E3M2, 2, 3, 32), (oracle.E3M2, oracle.E4M3, 3, 2, 64)])
def test_fp6_gemm_exact_rationals(ea, eb, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + ea + eb)
    aq, as_ = _rand(rng, M, K, ea)
    bq, bs = _rand(rng, N, K, eb)
    C, ABS = oracle.mx_gemm(aq, as_, ea, bq, bs, eb, M, N, K)
    X = _exact(aq, as_, ea, bq, bs, eb, M, N, K)
    for i in range(M):
        for j in range(N):
            assert abs(Fraction(C[i, j]) - X[i, j]) <= Fraction(K // 32) * Fraction(2) ** -52 * Fraction(ABS[i, j])


@pytest.mark.parametrize("elem", [oracle.E2M3, oracle.E3M2])
def test_fp6_packing_round_trip(elem):
    """Quantizing values already on the grid (scale 2^0) returns their codes,
    packed four to three bytes in the stated bit order."""
    rng = np.random.default_rng(9 + elem)
    f = FP6[elem]
    t = _table(elem)
    codes = rng.integers(0, 64, size=(17, 128))
    codes[:, ::32] = 2 ** (f["ebits"] + f["mbits"]) - 1   # every block holds the largest value
    vals = t[codes].astype(np.float32)
    q, s = oracle.quantize(vals, elem)
    # floor(log2(largest)) = emax, so every block's scale is 2^0 (byte 127)
    assert (s == 127).all()
    got = _unpack6(q, 128)
    # -0 and +0 both decode to zero; compare values, and codes away from zero
    assert np.array_equal(t[got], t[codes])
    nz = (codes & 31) != 0
    assert np.array_equal(got[nz], codes[nz])


def test_fp6_gemm_gate_detects_flipped_code():
    rng = np.random.default_rng(6)
    M, N, K = 16, 16, 512
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32)
    aq, as_ = oracle.quantize(a, oracle.E4M3)
    bq, bs = oracle.quantize(b, oracle.E2M3)
    C, ABS = oracle.mx_gemm(aq, as_, oracle.E4M3, bq, bs, oracle.E2M3, M, N, K)
    assert oracle.gate(C.astype(np.float32), C, ABS, K)["ok"]
    bq2 = bq.copy()
    bq2[5, 17] ^= 0x30   # two bits of one or two 6-bit codes
    C2, _ = oracle.mx_gemm(aq, as_, oracle.E4M3, bq2, bs, oracle.E2M3, M, N, K)
    assert not oracle.gate(C2.astype(np.float32), C, ABS, K)["ok"]
