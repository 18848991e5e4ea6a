"""Seeded sweep of mid-size MX products (the 4-wave tiled kernel and the
128 x 128 ping-pong; the 256 x 256 ping-pong needs at least 256 full tiles
and has its own cases) over the six float format pairs, through the C ABI,
against the oracle at the strict K-term bound on sampled elements.

Shapes from one fixed seed: M and N from 128 to 1300 (full 128- and
256-row tiles and ragged edges), K from 1024 to 4096 in steps of 32 (K % 128
== 0 with full 128-tiles takes the 128 x 128 ping-pong, the rest the tiled
kernel), format pairs E4M3 x E4M3, E4M3 x E2M1, E2M1 x E2M1, E5M2 x E5M2,
E4M3 x E5M2 and E5M2 x E4M3 (E2M1 operands: K a multiple of 64).  About 4000
random output elements per case are computed by the oracle; outputs start as
NaN canaries (every element must be written) and LDS is poisoned before every
GEMM.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_mxgemm_amd import inputs as mxin
from gpu_util import binding, mx_case, mx_sources, say

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=1202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = i % 6
        M = int(rng.integers(129, 1301))
        N = int(rng.integers(129, 1301))
        if rng.random() < 0.4:   # full 128- or 256-row tiles
            t = 256 if rng.random() < 0.5 else 128
            M, N = max(t, M // t * t), max(t, N // t * t)
        K = 32 * int(rng.integers(32, 129))
        if fmt in (1, 2):
            K -= K % 64
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
def test_tile_sweep(M, N, K, fmt):
    say("tile sweep", M, N, K, fmt)
    a32, b32 = mx_sources("mxfp8_2048", M, N, K, seed=M * 131 + N * 17 + K + fmt)
    pts = mxin.sample_points(M, N, 4000, seed=M + N + K)
    r, c = mx_case(a32, b32, fmt, points=pts)
    assert r["ok"], r
    assert not np.isnan(c).any(), "unwritten output elements"
