"""Pins for the oracle quantizer (CPU only).

The quantizer's rule: block exponent e = floor(log2(amax)) - emax_elem
(emax 8 for E4M3, 2 for E2M1), clamped to [-127, 127], scale byte e + 127;
elements x * 2^-e rounded to nearest-even and saturated (448 / 6).

Independent references used here: torch's float32 -> float8_e4m3fn cast (RNE,
non-saturating: only compared where no saturation happens), a brute-force
nearest-value search over the torch E4M3 value list and over the OCP E2M1 value
list with ties broken to the even code, closed forms for the scale byte, and
the saturation cases of the RIGEL summary (tests/golden/e4m3_saturation.txt).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden_rows

E4M3_VALUES = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _e2m1_values():
    rows = read_golden_rows("e2m1_values.txt")
    return np.array([float(v) for _, v in rows])


def _block_rows(values_per_block):
    """rows x K fp32 from a list of 32-element blocks (one block per row)."""
    return np.array(values_per_block, dtype=np.float32).reshape(len(values_per_block), 32)


def _nearest_even(v, table, nbits_mant_lsb_mask=1):
    """Brute force: the code whose value is nearest to v among finite,
    non-negative table entries; on a tie the code with an even LSB wins;
    above the largest finite value, the largest finite value."""
    a = abs(v)
    best = None
    for code, val in enumerate(table):
        if np.isnan(val) or val < 0 or (val == 0 and math.copysign(1, val) < 0):
            continue
        d = abs(val - a)
        if best is None or d < best[0] or (d == best[0] and (code & 1) == 0):
            best = (d, code)
    return best[1]


@pytest.mark.parametrize("t", [-20, -7, -1, 0, 1, 5, 30])
def test_scale_byte_closed_form_e4m3(t):
    rng = np.random.default_rng(t + 100)
    blocks = []
    expect = []
    for mant in [1.0, 1.25, 1.5, 1.999999, 1.0000001]:
        x = rng.uniform(-1, 1, 32).astype(np.float32) * np.float32(2.0 ** t)
        x[rng.integers(32)] = np.float32(mant * 2.0 ** t) * (1 if rng.random() < 0.5 else -1)
        blocks.append(x)
        amax = np.max(np.abs(x.astype(np.float64)))
        expect.append(math.frexp(amax)[1] - 1 - 8 + 127)
    q, s = oracle.quantize(_block_rows(blocks), oracle.E4M3)
    assert s[:, 0].tolist() == expect


def test_scale_byte_closed_form_e2m1():
    x = np.zeros((3, 32), dtype=np.float32)
    x[0, 5] = 6.0      # floor(log2 6) = 2 -> e = 0 -> byte 127
    x[1, 0] = -1.0     # 0 - 2 -> byte 125
    x[2, 31] = 0.75    # -1 - 2 -> byte 124
    q, s = oracle.quantize(x, oracle.E2M1)
    assert s[:, 0].tolist() == [127, 125, 124]


def test_zero_block_and_signed_zero():
    x = np.zeros((2, 32), dtype=np.float32)
    x[1, :] = -0.0
    q, s = oracle.quantize(x, oracle.E4M3)
    assert s[:, 0].tolist() == [0, 0]
    assert (q[0] == 0).all() and (q[1] == 0x80).all()
    q4, s4 = oracle.quantize(x, oracle.E2M1)
    assert (q4[0] == 0).all() and (q4[1] == 0x88).all()


def test_nonfinite_block_gets_nan_scale():
    x = np.ones((3, 64), dtype=np.float32)
    x[0, 3] = np.nan
    x[1, 40] = np.inf
    x[2, 63] = -np.inf
    q, s = oracle.quantize(x, oracle.E4M3)
    assert s.tolist() == [[255, 119], [119, 255], [119, 255]]
    assert (q[0, :32] == 0).all() and (q[1, 32:] == 0).all()


def test_e4m3_saturation_golden():
    rows = read_golden_rows("e4m3_saturation.txt")
    x = np.zeros((len(rows), 32), dtype=np.float32)
    for r, (val, _) in enumerate(rows):
        x[r, 7] = np.float32(float(val))
    q, s = oracle.quantize(x, oracle.E4M3)
    for r, (val, code) in enumerate(rows):
        assert s[r, 0] == 127, val
        assert q[r, 7] == int(code, 16), val


def test_e4m3_elements_match_torch_cast_where_unsaturated():
    rng = np.random.default_rng(7)
    rows = 512
    x = (rng.standard_normal((rows, 32)) * np.exp2(rng.integers(-30, 30, size=(rows, 1)))).astype(np.float32)
    # a few blocks with very small and very large spread
    x[:16] *= np.exp2(rng.integers(-20, 0, size=(16, 32))).astype(np.float32)
    q, s = oracle.quantize(x, oracle.E4M3)
    e = s[:, 0].astype(np.int64) - 127
    v = x.astype(np.float64) * np.exp2(-e)[:, None]          # exact
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    unsat = np.abs(v) <= 448.0
    assert unsat.mean() > 0.9
    assert np.array_equal(q[unsat], ref[unsat])
    sat = ~unsat
    assert np.array_equal(q[sat] & 0x7F, np.full(sat.sum(), 0x7E, dtype=np.uint8))


def test_e4m3_elements_match_bruteforce_nearest_even():
    rng = np.random.default_rng(8)
    # values straddling binade edges, subnormals, ties and the top of range
    vals = [0.0, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -9, 1.5 * 2.0 ** -9, 2.0 ** -6 - 2.0 ** -10,
            2.0 ** -6, 0.9375 * 2.0 ** -5, 1.0, 1.0625, 1.1875, 255.0, 256.0, 272.0, 304.0,
            447.0, 448.0, 455.0]
    vals += (rng.uniform(0, 448, 200)).tolist()
    vals += (np.exp2(rng.uniform(-12, 8.8, 300))).tolist()
    x = np.zeros((len(vals), 32), dtype=np.float32)
    x[:, 0] = 256.0          # fixes the block exponent at 0 (scale byte 127)
    x[:, 1] = np.array(vals, dtype=np.float32)
    x[:, 2] = -np.array(vals, dtype=np.float32)
    q, s = oracle.quantize(x, oracle.E4M3)
    assert (s[:, 0] == 127).all()
    for r in range(len(vals)):
        v = float(np.float32(vals[r]))
        c = _nearest_even(v, E4M3_VALUES)
        assert q[r, 1] == c, (v, q[r, 1], c)
        assert q[r, 2] == (c | 0x80), (v, q[r, 2], c)


def test_e2m1_elements_match_bruteforce_nearest_even():
    table = _e2m1_values()
    rng = np.random.default_rng(9)
    vals = [0.0, 0.24, 0.25, 0.26, 0.75, 1.25, 1.75, 2.5, 3.5, 4.99, 5.0, 5.01, 5.99, 6.0, 7.99]
    vals += rng.uniform(0, 8, 300).tolist()
    x = np.zeros((len(vals), 32), dtype=np.float32)
    x[:, 0] = 4.0            # block exponent 0
    x[:, 2] = np.array(vals, dtype=np.float32)
    x[:, 3] = -np.array(vals, dtype=np.float32)
    q, s = oracle.quantize(x, oracle.E2M1)
    assert (s[:, 0] == 127).all()
    lo = q[:, 1] & 0x0F   # k = 2 (even): low nibble of byte 1
    hi = q[:, 1] >> 4     # k = 3 (odd): high nibble of byte 1
    for r in range(len(vals)):
        v = float(np.float32(vals[r]))
        c = _nearest_even(v, table)
        assert lo[r] == c, (v, lo[r], c)
        assert hi[r] == (c | 0x8), (v, hi[r], c)


def test_e2m1_nibble_order():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.0   # code 2, even k -> low nibble
    x[0, 1] = 6.0   # code 7, odd k -> high nibble (block amax 6 -> e = 0)
    q, s = oracle.quantize(x, oracle.E2M1)
    assert q.shape == (1, 16)
    assert q[0, 0] == 0x72


def test_block_max_lands_in_top_binade():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((300, 256)) * np.exp2(rng.integers(-40, 40, size=(300, 1)))).astype(np.float32)
    q, s = oracle.quantize(x, oracle.E4M3)
    vals = np.abs(E4M3_VALUES[q]).reshape(300, 8, 32).max(axis=2)
    assert ((vals >= 256) & (vals <= 448)).all()
    q4, s4 = oracle.quantize(x, oracle.E2M1)
    t4 = _e2m1_values()
    codes = np.stack([q4 & 15, q4 >> 4], axis=-1).reshape(300, 256)
    v4 = np.abs(t4[codes]).reshape(300, 8, 32).max(axis=2)
    assert ((v4 >= 4) & (v4 <= 6)).all()


@pytest.mark.parametrize("elem", [oracle.E4M3, oracle.E2M1])
def test_requantize_is_idempotent(elem):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 128)) * np.exp2(rng.integers(-10, 10, size=(64, 4)).repeat(32, 1))).astype(np.float32)
    q, s = oracle.quantize(x, elem)
    scale = np.exp2(s.astype(np.float64) - 127).repeat(32, axis=1)
    if elem == oracle.E4M3:
        dec = E4M3_VALUES[q]
    else:
        t4 = _e2m1_values()
        dec = t4[np.stack([q & 15, q >> 4], axis=-1).reshape(64, 128)]
    xr = (dec * scale).astype(np.float32)
    q2, s2 = oracle.quantize(xr, elem)
    assert np.array_equal(s, s2)
    # -0 may appear where a tiny negative rounded to zero; compare values
    assert np.array_equal(q, q2)


def test_tiny_block_clamps_scale():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = np.float32(2.0 ** -149)  # smallest fp32 subnormal
    x[0, 1] = np.float32(2.0 ** -120)
    q, s = oracle.quantize(x, oracle.E4M3)
    assert s[0, 0] == 0       # e = -127
    # 2^-120 * 2^127 = 128 -> code 0x70 ; 2^-149 * 2^127 = 2^-22 -> rounds to 0
    assert q[0, 1] == 0x70 and q[0, 0] == 0x00
