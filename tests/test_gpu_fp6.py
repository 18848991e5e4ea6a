"""GPU parity of the FP6 element formats (E2M3, E3M2 codes with one UE8M0
scale per 32 K elements) through the C ABI, against the CPU oracle.

Quantizer: bit-exact, on normal data, on every fp32 mantissa at the
exponents where FP6 rounding changes regime (subnormal, normal, saturating
binades), and on special blocks.  GEMM (E4M3 activations x FP6 weights, fed
to the scaled MFMA's FP6 modes as stored, on the decode, split-K and tiled
kernels): the strict K-term bound per element, NaN positions identical; one
and several row blocks, more than 64 rows (the tiled kernel when K is a
multiple of 128, else the split-K kernel once per 64 rows), K not a multiple
of 128 or of 1024 (decode plus split-K remainder), K in chunks above 12288,
ragged N, and the decode workload at full size.  Outputs start as NaN
canaries and LDS is poisoned before every GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_mxgemm_amd import inputs as mxin
from gpu_util import binding, gpu_mx, gpu_quantize, model_gate, mx_case, mx_sources, say

pytestmark = pytest.mark.gpu

FMT = {oracle.E2M3: 8, oracle.E3M2: 9}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert binding().mxgemm_device_supported()
    yield


@pytest.mark.parametrize("elem", [oracle.E2M3, oracle.E3M2])
@pytest.mark.parametrize("rows,K", [(1, 32), (37, 96), (256, 256), (513, 4096)])
def test_fp6_quantize_bitexact(elem, rows, K):
    say("fp6 quantize", elem, rows, K)
    rng = np.random.default_rng(rows * 17 + K + elem)
    x = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-30, 30, size=(rows, K // 32))).repeat(32, 1)
         ).astype(np.float32)
    if rows > 1:
        x[0, :3] = [np.nan, 1.0, 2.0]   # a NaN block
        x[-1, :32] = 0.0                 # an all-zero block with a negative zero
        x[-1, 1] = -0.0
    if rows > 1 and K > 64:
        x[1, 40:43] = [np.inf, -0.0, 1e-42]   # an infinity block
    q, s = gpu_quantize(x, elem)
    qo, so = oracle.quantize(x, elem)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("elem", [oracle.E2M3, oracle.E3M2])
def test_fp6_quantize_every_mantissa(elem):
    """All 2^23 fp32 mantissas, both signs, at exponents across the
    regimes, with the block maximum fixed at 2^emax so the scale is 2^0:
    below half the subnormal step (rounds to zero or the first subnormal),
    the subnormal binades, a normal binade and the saturating top binade
    (E2M3: 7.5 .. 8 -> 7.5; E3M2: 28 .. 32 -> 28)."""
    say("fp6 quantize every mantissa", elem)
    if elem == oracle.E2M3:
        amax, ks = np.float32(4.0), (-4, -3, -1, 0, 2)
    else:
        amax, ks = np.float32(16.0), (-5, -4, -3, 1, 4)
    mant = np.arange(1 << 23, dtype=np.uint32)
    for k in ks:
        for sign in (0, 1):
            v = ((np.uint32(sign) << np.uint32(31)) | (np.uint32(k + 127) << np.uint32(23)) | mant).view(np.float32)
            v = np.concatenate([v, v[:(-len(v)) % 31]]).reshape(-1, 31)
            x = np.empty((v.shape[0], 32), dtype=np.float32)
            x[:, 0] = amax
            x[:, 1:] = v
            q, s = gpu_quantize(x, elem)
            qo, so = oracle.quantize(x, elem)
            assert np.array_equal(s.cpu().numpy(), so), (k, sign)
            assert np.array_equal(q.cpu().numpy(), qo), (k, sign)


# (M, N, K): one row block (1, 13, 16 rows), two and four, more than 64 rows
# (several split-K launches), K not a multiple of 128, ragged N.  With K a
# multiple of 1024 from 2048 and up to 64 rows the decode kernel takes the
# product: besides the shapes above, K in several chunks adding into C
# (16384 for one row block, 12288 with four: 3 chunks), K = 4160 (the
# decode kernel for 4096, the split-K kernel adds the rest), N = 1 and
# N < 16 (one ragged fragment)
FP6_SHAPES = [(1, 300, 2048), (16, 1001, 4096), (13, 250, 8192), (32, 300, 4096), (40, 777, 8192), (64, 500, 4096),
              (7, 1000, 1536), (33, 250, 96), (5, 28, 32), (64, 129, 256), (65, 300, 512), (200, 130, 1024),
              (2, 40, 16384), (64, 520, 12288), (9, 300, 4160), (1, 1, 2048), (3, 13, 3072),
              # decode line stages: K / 1024 = 12 in one launch with the 4-stage
              # ring (more fragments than CUs) and the 8-stage one, and 4
              (5, 4500, 12288), (3, 1000, 12288), (8, 4200, 4096),
              # more than 64 rows: the tiled kernel (K a multiple of 128; full
              # and ragged 128-tiles), and K = 2080 on the split-K kernel
              (256, 384, 2048), (130, 300, 1024), (300, 777, 4096), (100, 200, 2080)]

# measured above the strict K-term bound (one or three 128-element steps of
# the scaled MFMA, whose alignment term then exceeds K units: up to 6.2 x
# the strict bound, 0.026 x the model bound): gated with the step term, as
# the float and integer pairs' short-K cases
MODEL_CASES = {(33, 250, 96, 8), (33, 250, 96, 9), (5, 28, 32, 8), (5, 28, 32, 9)}


@pytest.mark.parametrize("fmt", [8, 9])
@pytest.mark.parametrize("M,N,K", FP6_SHAPES)
def test_fp6_gemm(fmt, M, N, K):
    say("fp6 gemm", fmt, M, N, K)
    a32, b32 = mx_sources("decode_16x28672x8192", M, N, K, seed=13 * M + N + K + fmt)
    r, c = mx_case(a32, b32, fmt, model=(M, N, K, fmt) in MODEL_CASES)
    assert r["ok"], r
    assert not np.isnan(c).any()


@pytest.mark.parametrize("fmt", [8, 9])
@pytest.mark.parametrize("M,N,K", [(4100, 4200, 384), (4096, 4352, 1024)])
def test_fp6_gemm_large_tiles(fmt, M, N, K):
    """Outputs with at least 256 tiles of 256 x 256 (the 256 x 256 tiled
    kernel), full and ragged edges, on sampled elements."""
    say("fp6 gemm large tiles", fmt, M, N, K)
    a32, b32 = mx_sources("decode_16x28672x8192", M, N, K, seed=17 * M + N + K + fmt)
    pts = mxin.sample_points(M, N, 20000, seed=M + N + K + fmt)
    r, c = mx_case(a32, b32, fmt, points=pts)
    assert r["ok"], r
    assert not np.isnan(c).any()


@pytest.mark.parametrize("fmt", [8, 9])
@pytest.mark.parametrize("M,N,K", [(8, 40, 2048), (100, 60, 256)])
def test_fp6_nan_scale(fmt, M, N, K):
    """A NaN scale byte in a row of A and in a row of B (FP6 has no NaN
    code) makes exactly that row / column NaN."""
    say("fp6 nan", fmt, M, N, K)
    ea, eb = oracle.E4M3, (oracle.E2M3 if fmt == 8 else oracle.E3M2)
    a32, b32 = mx_sources("decode_16x28672x8192", M, N, K, seed=M + N + K + fmt)
    qa, sa = gpu_quantize(a32, ea)
    qb, sb = gpu_quantize(b32, eb)
    sa[3, (K // 32) // 2] = 255
    sb[7, 1] = 255
    c = gpu_mx(qa, sa, qb, sb, fmt, M, N).cpu().numpy()
    qa_n, sa_n, qb_n, sb_n = (t.cpu().numpy() for t in (qa, sa, qb, sb))
    ref, ab, sm = oracle.mx_gemm(qa_n, sa_n, ea, qb_n, sb_n, eb, M, N, K, step_max=True)
    r = model_gate(c, ref, ab, sm, K, model=False)
    assert r["ok"], r
    want = np.zeros((M, N), dtype=bool)
    want[3, :] = True
    want[:, 7] = True
    assert np.array_equal(np.isnan(c), want)


@pytest.mark.parametrize("name,fmt", [("decode_e2m3_16x28672x8192", 8), ("decode_e3m2_16x28672x8192", 9)])
def test_fp6_decode_workload(name, fmt):
    """The decode workload with FP6 weights at full size, checked in full at
    the strict bound."""
    w = mxin.WORKLOADS[name]
    say("fp6 workload", name)
    a32, b32 = mxin.mx_sources(w)
    r, c = mx_case(a32, b32, fmt)
    assert r["ok"], r
    assert not np.isnan(c).any()
