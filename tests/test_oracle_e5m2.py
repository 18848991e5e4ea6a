"""Pins for the oracle's E5M2 element format (decode table and quantizer),
CPU only: torch's float8_e5m2 dtype (an independent implementation of the OCP
E5M2 format), hand-worked codes, a brute-force nearest-even search over the
format's values, and the scale rule's closed form."""
import numpy as np
import torch

import oracle

TORCH_E5 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()


def test_e5m2_table_matches_torch():
    t = oracle.e5m2_table()
    nan = np.isnan(TORCH_E5)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], TORCH_E5[~nan])


def test_e5m2_worked_codes():
    t = oracle.e5m2_table()
    assert t[0x3C] == 1.0 and t[0xBC] == -1.0
    assert t[0x7B] == 57344.0                       # largest finite: 1.75 * 2^15
    assert t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert all(np.isnan(t[c]) for c in (0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF))
    assert t[0x04] == 2.0 ** -14 and t[0x01] == 2.0 ** -16 and t[0x03] == 3 * 2.0 ** -16
    assert t[0x00] == 0.0 and np.signbit(t[0x80])


def _finite_values():
    t = oracle.e5m2_table()
    return np.unique(t[np.isfinite(t)])


def _nearest_even(v, grid, codes_of):
    """Brute force: the grid value nearest to v, ties to the even code."""
    d = np.abs(grid - v)
    best = np.flatnonzero(d == d.min())
    if best.size == 1:
        return grid[best[0]]
    even = [b for b in best if codes_of[grid[b]] % 2 == 0]
    return grid[even[0]]


def test_quantizer_scale_rule_and_elements():
    rng = np.random.default_rng(0)
    rows, K = 64, 256
    x = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-20, 20, (rows, 1)))).astype(np.float32)
    q, s = oracle.quantize(x, oracle.E5M2)
    t = oracle.e5m2_table()
    grid = _finite_values()
    pos_codes = {t[c]: c for c in range(0x00, 0x7C)}
    for r in range(rows):
        for b in range(K // 32):
            blk = x[r, 32 * b: 32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            e = int(np.floor(np.log2(amax))) - 15
            assert np.frexp(amax)[1] - 1 - 15 == e          # exact exponent, no float log2 trouble
            assert s[r, b] == e + 127
            v = np.ldexp(blk, -e)
            for k in range(32):
                code = q[r, 32 * b + k]
                a = abs(v[k])
                want = min(_nearest_even(a, grid[grid >= 0], pos_codes), 57344.0)
                assert t[code] == (-want if v[k] < 0 else want) or (want == 0 and t[code] == 0)
                if a <= 57344.0:      # where torch's cast cannot overflow it must agree
                    tc = torch.tensor([v[k]], dtype=torch.float32).to(torch.float8_e5m2).to(torch.float64).item()
                    assert t[code] == tc


def test_quantizer_saturates_the_block_maximum():
    # amax = 1.9 * 2^3: e = 3 - 15 = -12, v = 1.9 * 2^15 = 62259.2 lies past the
    # tie point 61440 between 57344 and 65536: saturates to 57344 (0x7B)
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1.9 * 8.0
    x[0, 1] = -1.9 * 8.0
    x[0, 2] = 1.0
    q, s = oracle.quantize(x, oracle.E5M2)
    assert s[0, 0] == 127 - 12
    assert q[0, 0] == 0x7B and q[0, 1] == 0xFB
    assert oracle.e5m2_table()[q[0, 2]] == 2.0 ** 12
    # a non-finite input makes the whole block NaN-scaled with zero codes
    x[0, 5] = np.inf
    q, s = oracle.quantize(x, oracle.E5M2)
    assert s[0, 0] == 255 and not q.any()
