"""Pins for the oracle's output step (bias, GELU, output type) - CPU only.

GELU(y) = y Phi(y) is pinned to textbook values of the standard normal
distribution function, to the identity GELU(y) - GELU(-y) = y, to scipy's
normal CDF, and its largest slope to the constant the gate uses.  The output
roundings are pinned to torch's float32 -> bfloat16 conversion and numpy's
float64 -> float16 conversion (both round to nearest even), plus hand-worked
ties, overflow and subnormal cases.
"""
import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

import oracle

# Phi(x) from standard normal tables
PHI = {1.0: 0.8413447460685429, 2.0: 0.9772498680518208, 3.0: 0.9986501019683699, 0.5: 0.6914624612740131}


def test_gelu_table_values():
    for x, phi in PHI.items():
        assert oracle.gelu(np.array([x]))[0] == pytest.approx(x * phi, rel=1e-15)
        assert oracle.gelu(np.array([-x]))[0] == pytest.approx(-x * (1.0 - phi), rel=1e-13)
    assert oracle.gelu(np.array([0.0]))[0] == 0.0
    assert oracle.gelu(np.array([10.0]))[0] == 10.0
    # far left tail: -10 Phi(-10), Phi(-10) = 7.619853024160527e-24
    assert oracle.gelu(np.array([-10.0]))[0] == pytest.approx(-10.0 * 7.619853024160527e-24, rel=1e-12)


def test_gelu_odd_part_identity():
    y = np.linspace(-8.0, 8.0, 4001)
    d = oracle.gelu(y) - oracle.gelu(-y)
    assert np.max(np.abs(d - y)) <= 4e-16 * np.max(np.abs(y))


def test_gelu_matches_scipy_normal_cdf():
    y = np.random.default_rng(0).uniform(-12.0, 12.0, 20000)
    ref = y * norm.cdf(y)
    got = oracle.gelu(y)
    assert np.all(np.abs(got - ref) <= 1e-14 * np.abs(y) + 1e-300)


def test_gelu_slope_bound():
    y = np.linspace(-10.0, 10.0, 200001)
    g = oracle.gelu(y)
    slope = np.abs(np.diff(g) / np.diff(y))
    assert slope.max() <= oracle.GELU_LIPSCHITZ
    # and it is the maximum, at y = sqrt(2): Phi(sqrt 2) + sqrt 2 phi(sqrt 2)
    s2 = math.sqrt(2.0)
    peak = norm.cdf(s2) + s2 * norm.pdf(s2)
    assert peak == pytest.approx(1.128904, abs=1e-6) and peak < oracle.GELU_LIPSCHITZ < peak + 1e-3


def test_gelu_nonfinite():
    g = oracle.gelu(np.array([np.inf, -np.inf, np.nan]))
    assert g[0] == np.inf and np.isnan(g[1]) and np.isnan(g[2])


def _torch_bf16(v32):
    return torch.from_numpy(np.asarray(v32, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    got = oracle.round_out(v.astype(np.float64), oracle.OUT_BF16)
    ref = _torch_bf16(v)
    assert np.array_equal(got, ref)


def test_bf16_rounding_worked_cases():
    r = lambda x: oracle.round_out(np.array([x], dtype=np.float64), oracle.OUT_BF16)[0]
    assert r(1.0) == 1.0
    assert r(1.0 + 2.0 ** -8) == 1.0                  # tie -> even (1.0)
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie -> even (1 + 2^-6)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    top = (2.0 - 2.0 ** -7) * 2.0 ** 127              # largest finite bf16
    assert r(top) == top
    assert r((2.0 - 2.0 ** -8) * 2.0 ** 127) == np.inf   # tie above the top -> even = infinity
    assert r(-(2.0 - 2.0 ** -8) * 2.0 ** 127 + 2.0 ** 100) == -top
    assert r(2.0 ** -133) == 2.0 ** -133              # smallest subnormal
    assert r(2.0 ** -134) == 0.0                      # tie -> even (0)
    assert r(3 * 2.0 ** -135) == 2.0 ** -133
    assert math.copysign(1.0, r(-0.0)) == -1.0
    assert np.isnan(r(np.nan))


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.uniform(-9, 5, 50000),
                        [65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, -0.0, 1.0 + 2.0 ** -11]])
    got = oracle.round_out(v, oracle.OUT_F16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)
    assert got[-3] == 5.960464477539063e-08 and got[-1] == 1.0  # 3*2^-26 -> 2^-24; 1 + 2^-11 (tie) -> 1


def test_epilogue_bias_and_gelu():
    c = np.array([1.0, 2.0, -3.0])
    cols = np.array([0, 1, 1])
    bias = np.array([0.5, -1.0], dtype=np.float32)
    assert np.array_equal(oracle.epilogue(c, cols, bias, oracle.ACT_NONE), [1.5, 1.0, -4.0])
    g = oracle.epilogue(c, cols, bias, oracle.ACT_GELU)
    assert g[1] == pytest.approx(PHI[1.0], rel=1e-15)
    assert np.array_equal(oracle.epilogue(c, cols, None, oracle.ACT_NONE), c)


def test_epilogue_gate_controls():
    rng = np.random.default_rng(3)
    n = 2000
    c = rng.standard_normal(n) * 4
    ab = np.abs(c) + 1.0
    cols = rng.integers(0, 64, n)
    bias = rng.standard_normal(64).astype(np.float32)
    ref = oracle.epilogue(c, cols, bias, oracle.ACT_GELU)
    out = oracle.round_out(ref, oracle.OUT_BF16)
    assert oracle.epilogue_gate(out, c, ab, 256, cols, bias, oracle.ACT_GELU, oracle.OUT_BF16)["ok"]
    bad = out.copy()
    bad[7] = oracle.round_out(np.array([ref[7] * (1 + 2.0 ** -5) + 0.1]), oracle.OUT_BF16)[0]
    assert not oracle.epilogue_gate(bad, c, ab, 256, cols, bias, oracle.ACT_GELU, oracle.OUT_BF16)["ok"]
    nan = out.copy()
    nan[3] = np.nan
    assert oracle.epilogue_gate(nan, c, ab, 256, cols, bias, oracle.ACT_GELU, oracle.OUT_BF16)["nan_mismatch"] == 1
    # a dropped bias is caught
    nob = oracle.round_out(oracle.epilogue(c, cols, None, oracle.ACT_GELU), oracle.OUT_BF16)
    assert not oracle.epilogue_gate(nob, c, ab, 256, cols, bias, oracle.ACT_GELU, oracle.OUT_BF16)["ok"]


def test_epilogue_gate_overflow_to_infinity():
    # 1e30 exceeds fp16: the exact value rounds to +inf, which the output must be
    c = np.array([1e30, -1e30, 1.0])
    cols = np.zeros(3, dtype=np.int64)
    ok = np.array([np.inf, -np.inf, 1.0])
    assert oracle.epilogue_gate(ok, c, np.zeros(3), 0, cols, None, oracle.ACT_NONE, oracle.OUT_F16)["ok"]
    bad = np.array([65504.0, -np.inf, 1.0])
    assert oracle.epilogue_gate(bad, c, np.zeros(3), 0, cols, None, oracle.ACT_NONE, oracle.OUT_F16)["inf_mismatch"] == 1
    # in bf16 the same values are finite
    fin = oracle.round_out(c, oracle.OUT_BF16)
    assert np.isfinite(fin).all()
    assert oracle.epilogue_gate(fin, c, np.zeros(3), 0, cols, None, oracle.ACT_NONE, oracle.OUT_BF16)["ok"]
