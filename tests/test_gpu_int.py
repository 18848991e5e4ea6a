"""GPU parity of the integer block formats (INT4, INT2 codes with one UE8M0
scale per 32 K elements) through the C ABI, against the CPU oracle.

Quantizer: bit-exact, on normal data, on every fp32 mantissa at the
exponents where integer rounding changes regime, and on special blocks.
GEMM (E4M3 activations x INT4 / INT2 weights, the weights remapped in
registers to E4M3 / E2M1 MFMA operands): the strict K-term bound per
element, NaN positions identical; the decode kernel (one launch, K chunks,
two row blocks, decode + split-K remainder), the split-K kernel, and more
than 64 rows (the split-K kernel once per 64 rows).  Outputs start as NaN
canaries and LDS is poisoned before every GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_mxgemm_amd import inputs as mxin
from gpu_util import binding, gpu_mx, gpu_quantize, model_gate, mx_case, mx_sources, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert binding().mxgemm_device_supported()
    yield


@pytest.mark.parametrize("elem", [oracle.INT4, oracle.INT2])
@pytest.mark.parametrize("rows,K", [(1, 32), (37, 96), (256, 256), (513, 4096)])
def test_int_quantize_bitexact(elem, rows, K):
    say("int quantize", elem, rows, K)
    rng = np.random.default_rng(rows * 13 + K + elem)
    x = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-30, 30, size=(rows, K // 32))).repeat(32, 1)
         ).astype(np.float32)
    x[0, :3] = [np.nan, 1.0, 2.0] if rows > 1 else x[0, :3]
    q, s = gpu_quantize(x, elem)
    qo, so = oracle.quantize(x, elem)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("elem", [oracle.INT4, oracle.INT2])
def test_int_quantize_every_mantissa(elem):
    """All 2^23 fp32 mantissas, both signs, at every exponent from the
    round-to-zero edge to saturation, with the block maximum fixed so the
    scale is 2^0: INT4 (block maximum 4) at 2^-2 .. 2^2, INT2 (block maximum
    1) at 2^-2 .. 2^0; ties at every half integer and both saturation
    edges (7.5 .. 8 -> +7 / -8; 1.5 .. 2 -> +1 / -2)."""
    say("int quantize every mantissa", elem)
    amax, ks = (np.float32(4.0), (-2, -1, 0, 1, 2)) if elem == oracle.INT4 else (np.float32(1.0), (-2, -1, 0))
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


# (M, N, K): decode kernel one launch (K 2048 .. 8192 and, for INT4, 14336 =
# the per-launch maximum), odd K / 1024 (uneven wave split for INT4), two and
# four row blocks, K chunks adding into C, decode + split-K remainder, the
# split-K kernel (K not a multiple of 1024, short K), more than 64 rows (the
# tiled kernel: full and ragged tiles, a partial last slice)
INT_SHAPES = [(1, 300, 2048), (16, 1001, 4096), (13, 250, 8192), (3, 64, 8192), (16, 1000, 3072), (9, 5000, 5120),
              (17, 1001, 8192), (32, 300, 4096), (40, 777, 8192), (64, 500, 4096), (16, 1000, 14336),
              (5, 300, 32768), (16, 700, 11008), (7, 1000, 1536), (33, 250, 96), (5, 28, 32), (64, 129, 256),
              (65, 300, 512), (200, 130, 1024), (256, 384, 2048), (130, 257, 1056), (100, 300, 2080)]


# measured above the strict K-term bound (one or three 128-element steps of
# the scaled MFMA, whose alignment term then exceeds K units): gated with the
# step term, as the float pairs' short-K cases
MODEL_CASES = {(33, 250, 96, 7), (5, 28, 32, 7)}


@pytest.mark.parametrize("fmt", [6, 7])
@pytest.mark.parametrize("M,N,K", INT_SHAPES)
def test_int_gemm(fmt, M, N, K):
    say("int gemm", fmt, M, N, K)
    a32, b32 = mx_sources("decode_16x28672x8192", M, N, K, seed=11 * M + N + K + fmt)
    r, c = mx_case(a32, b32, fmt, model=(M, N, K, fmt) in MODEL_CASES)
    assert r["ok"], r
    assert not np.isnan(c).any()


@pytest.mark.parametrize("fmt", [6, 7])
@pytest.mark.parametrize("M,N,K", [(4100, 4200, 384), (4096, 4352, 1056)])
def test_int_gemm_large_tiles(fmt, M, N, K):
    """Outputs with at least 256 tiles of 256 x 256 (the 256 x 256 tiled
    kernel), ragged edges and a partial last K slice, on sampled elements."""
    say("int gemm large tiles", fmt, M, N, K)
    a32, b32 = mx_sources("decode_16x28672x8192", M, N, K, seed=13 * M + N + K + fmt)
    pts = mxin.sample_points(M, N, 20000, seed=M + N + K + fmt)
    r, c = mx_case(a32, b32, fmt, points=pts)
    assert r["ok"], r
    assert not np.isnan(c).any()


@pytest.mark.parametrize("fmt", [6, 7])
@pytest.mark.parametrize("M,N,K", [(8, 40, 2048), (40, 520, 8192), (13, 40, 4608), (100, 60, 256)])
def test_int_nan_scale(fmt, M, N, K):
    """A NaN scale byte in a row of A and in a row of B (the integer codes
    have no NaN) makes exactly that row / column NaN."""
    say("int nan", fmt, M, N, K)
    ea, eb = oracle.E4M3, (oracle.INT4 if fmt == 6 else oracle.INT2)
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


@pytest.mark.parametrize("name,fmt", [("decode_int4_16x28672x8192", 6), ("decode_int2_16x28672x8192", 7)])
def test_int_decode_workload(name, fmt):
    """The decode workload with integer weights at full size, checked in
    full at the strict bound."""
    w = mxin.WORKLOADS[name]
    say("int workload", name)
    a32, b32 = mxin.mx_sources(w)
    r, c = mx_case(a32, b32, fmt)
    assert r["ok"], r
    assert not np.isnan(c).any()
