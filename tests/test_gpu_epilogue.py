"""GPU parity of the output step: the stand-alone epilogue kernel and the
epilogue fused into every MX GEMM kernel (bias, GELU, fp32 / bf16 / fp16 C).

* Conversions and the bias add are exact operations on fp32 inputs, so the
  epilogue kernel must match them bit for bit (torch's RNE conversions, numpy's
  float32 add).
* GELU is checked against the oracle's float64 y Phi(y) within the error its
  evaluation is allowed (oracle.epilogue_gate).
* The fused GEMM must equal mxgemm_run followed by mxgemm_epilogue bit for bit
  (the same fp32 accumulators through the same device arithmetic), and match
  the oracle through epilogue_gate; with no bias, no activation and fp32
  output it must equal mxgemm_run.  (Exception: decode shapes that the fp32
  path splits into K chunks take another schedule for 16-bit outputs; those
  are held to the oracle only.)
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_precision_mxgemm_amd import inputs as mxin
from gpu_util import FMT_ELEMS, MFMA_STEP_KAPPA, binding, poison_lds, gpu_quantize, mx_sources, say, to_dev

pytestmark = pytest.mark.gpu

OUT_DT = {oracle.OUT_F32: torch.float32, oracle.OUT_BF16: torch.bfloat16, oracle.OUT_F16: torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert binding().mxgemm_device_supported()
    yield


def _vals(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).cpu().numpy()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


def _special_matrix(rows=64, cols=1028, seed=0):
    """fp32 values over the whole range: random bit patterns, random normals,
    ties for the 16-bit formats, overflow and subnormal cases, +-0, +-inf,
    NaN.  cols is not a multiple of 8, so the scalar tail runs too."""
    rng = np.random.default_rng(seed)
    n = rows * cols
    bits = rng.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32).copy()
    x[: n // 3] = (rng.standard_normal(n // 3) * 10.0 ** rng.uniform(-6, 6, n // 3)).astype(np.float32)
    spec = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 65519.0, 65520.0,
                     3.3895314e38, 2.0 ** -133, 2.0 ** -134, 2.0 ** -25, 1.0 + 2.0 ** -11, 6e-8],
                    dtype=np.float32)
    x[n // 3: n // 3 + spec.size] = spec
    return x.reshape(rows, cols)


@pytest.mark.parametrize("out_type", [oracle.OUT_F32, oracle.OUT_BF16, oracle.OUT_F16])
def test_epilogue_conversion_is_exact(out_type):
    say("epilogue conversion", out_type)
    b = binding()
    x = _special_matrix()
    y = b.mxgemm_epilogue(to_dev(x), None, b.ACT_NONE, out_type)
    torch.cuda.synchronize()
    ref = torch.from_numpy(x).to(OUT_DT[out_type])   # torch CPU: round to nearest even
    got = y.cpu()
    nan = torch.isnan(ref).numpy()
    assert np.array_equal(torch.isnan(got).numpy(), nan)
    assert np.array_equal(_bits(got)[~nan], _bits(ref)[~nan])
    # the oracle's rounding agrees as well (values)
    with np.errstate(invalid="ignore"):
        assert np.array_equal(np.nan_to_num(_vals(y), nan=7.0),
                              np.nan_to_num(oracle.round_out(x.astype(np.float64), out_type), nan=7.0))


def test_epilogue_bias_add_is_exact():
    say("epilogue bias")
    b = binding()
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((37, 1001)) * 100).astype(np.float32)
    bias = rng.standard_normal(1001).astype(np.float32)
    y = b.mxgemm_epilogue(to_dev(x), to_dev(bias), b.ACT_NONE, b.OUT_F32)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint32), (x + bias[None, :]).view(np.uint32))


@pytest.mark.parametrize("out_type", [oracle.OUT_F32, oracle.OUT_BF16, oracle.OUT_F16])
def test_epilogue_gelu_against_oracle(out_type):
    say("epilogue gelu", out_type)
    b = binding()
    grid = np.linspace(-12.0, 12.0, 1 << 20, dtype=np.float32)
    extra = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -130, 300.0, -300.0, 1e30, -1e30, np.inf, np.nan,
                      np.float32(np.sqrt(2.0))], dtype=np.float32)
    x = np.concatenate([grid, extra, np.zeros(4, np.float32)]).reshape(-1, 4)   # N = 4: one vector per row
    y = b.mxgemm_epilogue(to_dev(x), None, b.ACT_GELU, out_type)
    torch.cuda.synchronize()
    got = _vals(y).ravel()
    c = x.astype(np.float64).ravel()
    cols = np.tile(np.arange(4), x.shape[0])
    r = oracle.epilogue_gate(got, c, np.zeros_like(c), 0, cols, None, oracle.ACT_GELU, out_type)
    say("  ", r)
    assert r["ok"], r
    assert np.isnan(got[np.flatnonzero(np.isnan(c))]).all()


# (workload recipe, M, N, K, fmt): the ping-pong kernel (>= 256 full tiles,
# fp8 and fp4 x fp4; with 272 tiles, a second tile per workgroup; K = 1152
# ends with a partial scale group), the 128 x 128 split-K ping-pong (full
# 128-tiles), the
# 128 x 128 tiled kernel (ragged), a ragged shape with
# >= 256 tiles (plain fp32 takes the 256 x 256 tiled kernel, a general
# epilogue the 128 x 128 one), the decode kernel (1, 3 row blocks; two
# K chunks at K = 8192 for 33 rows, 20480 and, with E4M3 weights, 14336,
# where 16-bit outputs take two row launches or the split-K kernel instead;
# K = 4608 split between the decode and split-K kernels; E2M3 / E3M2 weights
# on the same paths) and the split-K skinny kernel.
CASES = [("mxfp8_8192", 4096, 4096, 256, 0, 20000), ("mxfp8_2048", 4096, 4352, 256, 2, 20000),
         ("mxfp8_2048", 4096, 4352, 1024, 4, 20000), ("mxfp8_2048", 4096, 4352, 1152, 0, 20000),
         ("mxfp8_2048", 512, 640, 384, 0, None), ("mxfp8_2048", 512, 640, 384, 4, None),
         ("mxfp8_2048", 300, 257, 512, 0, None), ("prefill_8192x14336x4096", 520, 530, 1056, 1, None),
         ("mxfp8_2048", 4100, 4100, 128, 0, 20000), ("decode_16x28672x8192", 16, 1000, 2048, 1, None),
         ("decode_16x28672x8192", 48, 1000, 4096, 0, None), ("decode_16x28672x8192", 33, 1001, 8192, 1, None),
         ("decode_16x28672x8192", 40, 512, 1536, 0, None), ("decode_16x28672x8192", 7, 1003, 1536, 1, None),
         ("decode_16x28672x8192", 17, 1001, 20480, 1, None), ("decode_16x28672x8192", 16, 600, 14336, 0, None),
         ("decode_16x28672x8192", 13, 1001, 4608, 1, None), ("decode_16x28672x8192", 16, 1000, 4096, 8, None),
         ("decode_16x28672x8192", 33, 1001, 8192, 9, None), ("decode_16x28672x8192", 13, 1001, 4608, 8, None),
         ("decode_16x28672x8192", 17, 600, 14336, 9, None), ("decode_16x28672x8192", 200, 300, 1024, 8, None),
         ("decode_16x28672x8192", 130, 257, 2048, 9, None), ("decode_16x28672x8192", 150, 260, 1056, 6, None),
         ("decode_16x28672x8192", 140, 270, 2080, 7, None)]

EPILOGUES = [(True, oracle.ACT_GELU, oracle.OUT_BF16), (True, oracle.ACT_NONE, oracle.OUT_F16),
             (False, oracle.ACT_GELU, oracle.OUT_F32), (True, oracle.ACT_GELU, oracle.OUT_F16)]


# cases measured to exceed the strict K-term bound at K <= 384, where the
# scaled-MFMA step term (test_gpu_mfma_error.py) is added to the GEMM's bound
MODEL_CASES = {("mxfp8_2048", 512, 640, 384, 0), ("mxfp8_2048", 512, 640, 384, 4), ("mxfp8_2048", 4100, 4100, 128, 0)}


@pytest.mark.parametrize("name,M,N,K,fmt,npts", CASES)
def test_fused_gemm(name, M, N, K, fmt, npts):
    say("fused gemm", name, M, N, K, fmt)
    model = (name, M, N, K, fmt) in MODEL_CASES
    b = binding()
    a32, b32 = mx_sources(name, M, N, K, seed=M + 3 * N + K + fmt)
    ea, eb = FMT_ELEMS[fmt]
    qa, sa = gpu_quantize(a32, ea)
    qb, sb = gpu_quantize(b32, eb)
    qa_o, sa_o = oracle.quantize(a32, ea)
    qb_o, sb_o = oracle.quantize(b32, eb)
    assert np.array_equal(qa.cpu().numpy(), qa_o) and np.array_equal(qb.cpu().numpy(), qb_o)
    assert np.array_equal(sa.cpu().numpy(), sa_o) and np.array_equal(sb.cpu().numpy(), sb_o)
    rng = np.random.default_rng(N)
    bias_np = rng.standard_normal(N).astype(np.float32)
    bias = to_dev(bias_np)
    plain = b.mxgemm_run(qa, sa, qb, sb, fmt)
    same = b.mxgemm_run_fused(qa, sa, qb, sb, fmt)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int32), same.view(torch.int32)), "plain fused output differs from mxgemm_run"
    if npts is None:
        I, J = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        I, J = I.ravel(), J.ravel()
        ref, ab, sm = oracle.mx_gemm(qa_o, sa_o, ea, qb_o, sb_o, eb, M, N, K, step_max=True)
        ref, ab, sm = ref.ravel(), ab.ravel(), sm.ravel()
    else:
        I, J = mxin.sample_points(M, N, npts)
        ref, ab, sm = oracle.mx_gemm(qa_o, sa_o, ea, qb_o, sb_o, eb, M, N, K, points=(I, J), step_max=True)
    kappa = MFMA_STEP_KAPPA if model else 0.0
    # With fp32 C the decode kernel covers all M rows in one launch per K
    # chunk, as many chunks as the A operands of M / 16 row blocks need, and
    # keeps the running sum in C; a 16-bit C takes all of K per launch (fewer
    # rows each) or, beyond one launch's K, the split-K kernel.  Where fp32
    # C needs several chunks, the two sum in another order (both are checked
    # against the oracle).
    # With fp32 C and up to 16 rows, K not a multiple of 1024 (above 2048)
    # also splits: the decode kernel takes the multiples of 1024, the split-K
    # kernel adds the rest; a 16-bit C takes the split-K kernel for all of K.
    blocks = (M + 15) // 16
    limit = (16 if fmt == 1 else 12) if blocks <= 1 else 8 if blocks <= 2 else 4
    decode_rows = fmt in (0, 1, 8, 9) and M <= 64
    chunked = decode_rows and ((K % 1024 == 0 and K >= 2048 and K // 1024 > limit) or
                               (M <= 16 and K % 1024 != 0 and K - K % 1024 >= 2048))
    for use_bias, act, out_type in EPILOGUES:
        bb = bias if use_bias else None
        poison_lds()
        fused = b.mxgemm_run_fused(qa, sa, qb, sb, fmt, bias=bb, act=act, out_type=out_type)
        dec = b.mxgemm_epilogue(plain, bb, act, out_type)
        torch.cuda.synchronize()
        if not (chunked and out_type != oracle.OUT_F32):
            assert np.array_equal(_bits(fused), _bits(dec)), ("fused differs from the decomposed path", use_bias,
                                                           act, out_type)
        got = _vals(fused)[I, J]
        r = oracle.epilogue_gate(got, ref, ab, K, J, bias_np if use_bias else None, act, out_type,
                                 step_max=sm, kappa=kappa)
        rm = oracle.epilogue_gate(got, ref, ab, K, J, bias_np if use_bias else None, act, out_type,
                                  step_max=sm, kappa=MFMA_STEP_KAPPA)
        say("  ", use_bias, act, out_type, r, "model max ratio %.4g" % rm["max_ratio"])
        assert r["ok"], (use_bias, act, out_type, r)


def test_fused_gemm_graph_replay():
    """The fused path captured in a HIP graph and replayed with other work
    in between: every replay reproduces the eager bits."""
    say("fused graph replay")
    b = binding()
    M, N, K = 4096, 4096, 256
    a32, b32 = mx_sources("mxfp8_8192", M, N, K, seed=9)
    qa, sa = gpu_quantize(a32, oracle.E4M3)
    qb, sb = gpu_quantize(b32, oracle.E4M3)
    bias = to_dev(np.random.default_rng(1).standard_normal(N).astype(np.float32))
    run = lambda out: b.mxgemm_run_fused(qa, sa, qb, sb, 0, bias=bias, act=b.ACT_GELU, out_type=b.OUT_BF16, out=out)
    eager = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    run(eager)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    run(out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for rep in range(3):
        out.fill_(float("nan"))
        b.mxgemm_run(qa, sa, qb, sb, 0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), _bits(eager)), rep
    del g
