"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  Quantizer bytes are compared in full (bit-exact); GEMM
outputs are compared on sampled points (every output tile's corners and
centre, the last row and column, plus random points), each against the float64
oracle, with the bound |C - C_ref| <= K * 2^-24 * sum_k |a_ik b_jk| and NaN
positions identical.  Outputs start as NaN canaries.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_mxgemm_amd import inputs as mxin
from gpu_util import binding, mx_case, nan_canary, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert binding().mxgemm_device_supported()
    yield


MX_WORKLOADS = [("mxfp8_256", 0, None), ("mxfp8_2048", 0, 30000), ("prefill_8192x14336x4096", 0, 30000),
                ("prefill_mxfp4_8192x14336x4096", 2, 30000), ("decode_16x28672x8192", 1, None),
                ("mxfp8_8192", 0, 30000), ("mxfp8xbf8_8192", 4, 30000),
                ("prefill_e2m3_8192x14336x4096", 8, 30000), ("prefill_int4_8192x14336x4096", 6, 30000),
                ("prefill_int2_8192x14336x4096", 7, 30000)]


@pytest.mark.parametrize("name,fmt,npts", MX_WORKLOADS)
def test_mx_workload(name, fmt, npts):
    w = mxin.WORKLOADS[name]
    say("workload", name, w.M, w.N, w.K)
    a32, b32 = mxin.mx_sources(w)
    pts = None if npts is None else mxin.sample_points(w.M, w.N, npts)
    r, c = mx_case(a32, b32, fmt, points=pts)   # the strict K-term bound
    say("  gate", r)
    assert r["ok"], r
    assert not np.isnan(c).any(), "unwritten outputs"


def test_fp16_pair_2048():
    """The paired fp16 run of the 2048^3 workload (same fp32 sources, N x K)."""
    w = mxin.WORKLOADS["mxfp8_2048"]
    say("fp16 pair 2048")
    a16, b16 = mxin.fp16_sources(w, b_is_nk=True)
    out = nan_canary(w.M, w.N)
    binding().fp16gemm_run(to_dev(a16), to_dev(b16), True, out=out)
    torch.cuda.synchronize()
    c = out.cpu().numpy()
    pts = mxin.sample_points(w.M, w.N, 20000)
    ref, ab = oracle.fp16_gemm(a16.view(np.uint16), b16.view(np.uint16), w.M, w.N, w.K, 1, points=pts)
    r = oracle.gate(c[pts[0], pts[1]], ref, ab, w.K)
    assert r["ok"], r
    assert not np.isnan(c).any()


def test_fp16_pair_8192():
    w = mxin.WORKLOADS["mxfp8_8192"]
    say("fp16 pair 8192")
    a16, b16 = mxin.fp16_sources(w, b_is_nk=True)
    out = nan_canary(w.M, w.N)
    binding().fp16gemm_run(to_dev(a16), to_dev(b16), True, out=out)
    torch.cuda.synchronize()
    c = out.cpu().numpy()
    pts = mxin.sample_points(w.M, w.N, 20000)
    ref, ab = oracle.fp16_gemm(a16.view(np.uint16), b16.view(np.uint16), w.M, w.N, w.K, 1, points=pts)
    r = oracle.gate(c[pts[0], pts[1]], ref, ab, w.K)
    assert r["ok"], r
    assert not np.isnan(c).any()
