"""Every entry point captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed several times, with eager launches and synchronizations of the
program between the replays: each replay must reproduce the eager result bit
for bit.  The library records no memsets and allocates nothing per call, so
its launches are capturable as they are; bench.py times the short
configurations this way.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import binding, gpu_quantize, mx_sources, say, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert binding().mxgemm_device_supported()
    yield


def _check_replays(run, make_out, other):
    """run(out) launches into out; other() is unrelated eager work."""
    eager = make_out()
    run(eager)
    torch.cuda.synchronize()
    ref = eager.cpu().numpy().copy()
    out = make_out()
    run(out)  # warm-up outside the capture (first-call device queries)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for rep in range(REPLAYS):
        out.fill_(float("nan")) if out.dtype == torch.float32 else out.fill_(0xA5)
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), "replay %d differs from the eager result" % rep
    del g


def _mx_operands(name, M, N, K, fmt, seed):
    a32, b32 = mx_sources(name, M, N, K, seed=seed)
    ea, eb = {0: (oracle.E4M3, oracle.E4M3), 1: (oracle.E4M3, oracle.E2M1), 2: (oracle.E2M1, oracle.E2M1)}[fmt]
    qa, sa = gpu_quantize(a32, ea)
    qb, sb = gpu_quantize(b32, eb)
    return qa, sa, qb, sb


# ping-pong (256 tiles of 256 x 256), 128 x 128 tiled (ragged N), decode
# (one launch; two K chunks adding into C, for 40 rows at K = 8192 and for
# K = 20480 / 14336 beyond one launch's range) and split-K skinny kernels
@pytest.mark.parametrize("name,M,N,K,fmt", [("mxfp8_8192", 4096, 4096, 256, 0),
                                            ("mxfp8_2048", 512, 384, 512, 0),
                                            ("decode_16x28672x8192", 16, 1000, 2048, 1),
                                            ("decode_16x28672x8192", 48, 1000, 4096, 0),
                                            ("decode_16x28672x8192", 40, 1000, 8192, 1),
                                            ("decode_16x28672x8192", 16, 1000, 20480, 1),
                                            ("decode_16x28672x8192", 16, 600, 14336, 0),
                                            ("decode_16x28672x8192", 40, 512, 1536, 0)])
def test_mx_gemm_graph_replay(name, M, N, K, fmt):
    say("graph replay mx", name, M, N, K, fmt)
    b = binding()
    qa, sa, qb, sb = _mx_operands(name, M, N, K, fmt, seed=M + N + K)
    scratch = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    _check_replays(lambda out: b.mxgemm_run(qa, sa, qb, sb, fmt, out=out),
                   lambda: torch.empty((M, N), dtype=torch.float32, device="cuda:0"),
                   lambda: b.mxgemm_run(qa, sa, qb, sb, fmt, out=scratch))


@pytest.mark.parametrize("M,N,K,b_is_nk", [(4096, 4096, 128, True), (256, 384, 512, False)])
def test_fp16_gemm_graph_replay(M, N, K, b_is_nk):
    say("graph replay fp16", M, N, K, b_is_nk)
    b = binding()
    rng = np.random.default_rng(M + N + K)
    a16 = to_dev(rng.uniform(-1, 1, (M, K)).astype(np.float16))
    b16 = to_dev(rng.uniform(-1, 1, (N, K) if b_is_nk else (K, N)).astype(np.float16))
    scratch = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    _check_replays(lambda out: b.fp16gemm_run(a16, b16, b_is_nk, out=out),
                   lambda: torch.empty((M, N), dtype=torch.float32, device="cuda:0"),
                   lambda: b.fp16gemm_run(a16, b16, b_is_nk, out=scratch))


@pytest.mark.parametrize("elem", [oracle.E4M3, oracle.E2M1])
def test_quantize_graph_replay(elem):
    say("graph replay quantize", elem)
    b = binding()
    rows, K = 300, 1024
    x = to_dev(np.random.default_rng(3).standard_normal((rows, K)).astype(np.float32))
    s_out = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda:0")
    qbytes = K if elem == oracle.E4M3 else K // 2

    def run(q):
        b.mxgemm_quantize(x, elem, q=q, s=s_out)

    _check_replays(run, lambda: torch.empty((rows, qbytes), dtype=torch.uint8, device="cuda:0"),
                   lambda: b.mxgemm_quantize(x * 2.0, elem))
