"""Seeded sweep of decode-shaped MX products (few activation rows against a
weight matrix) over every weight element type, through the C ABI, against the
oracle element by element at the strict K-term bound.

The shapes are drawn from one fixed seed: M from 1 to 40 (one to three blocks
of 16 rows, ragged), N ragged from 17 to 1500, K a multiple of 1024 from 2048
to 16384, sometimes plus a remainder of 32 to 992 (decode kernel plus the
split-K kernel for the rest), and the weight type E4M3, E2M1, INT4, INT2, E2M3
or E3M2.  So the draw mixes the decode kernel's K chunking, row-block counts,
ring depths, FP6 line and 96-byte stages and the split-K remainder in
combinations the hand-picked cases do not list.  Operands are the decode
workload's N(0, 1) recipe; outputs start as NaN canaries and LDS is poisoned
before every GEMM.
"""
import numpy as np
import pytest
import torch

from gpu_util import binding, mx_case, mx_sources, say

pytestmark = pytest.mark.gpu


def _cases(n=30, seed=20261202):
    rng = np.random.default_rng(seed)
    fmts = [0, 1, 6, 7, 8, 9]
    out = []
    for i in range(n):
        fmt = fmts[i % len(fmts)]
        M = int(rng.integers(1, 41))
        N = int(rng.integers(17, 1501))
        K = 1024 * int(rng.integers(2, 17))
        if rng.random() < 0.3:
            K += 32 * int(rng.integers(1, 32))
        out.append((M, N, K, fmt))
    return out


CASES = _cases()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert binding().mxgemm_device_supported()
    yield


@pytest.mark.parametrize("M,N,K,fmt", CASES)
def test_decode_sweep(M, N, K, fmt):
    say("decode sweep", M, N, K, fmt)
    a32, b32 = mx_sources("decode_16x28672x8192", M, N, K, seed=M * 7919 + N * 31 + K + fmt)
    r, c = mx_case(a32, b32, fmt)
    assert r["ok"], r
    assert not np.isnan(c).any()
