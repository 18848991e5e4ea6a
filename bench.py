"""Benchmark of the MX GEMM path on one MI355X.

Prints ONE JSON line on stdout.  The step is one mxgemm_run of the MXFP8
8192 x 8192 x 8192 workload (E4M3 codes, UE8M0 scale per 32 K elements, fp32
output) on operands already resident in HBM; `value` is its throughput in
TFLOP/s (2*M*N*K per step) over exactly K timed steps after W warm-up steps.
The same run measures every workload of the path (the paired fp16 GEMMs and
the fp8/fp16 ratios, 2048^3, 1024^3 fp16, 256^3, the LLM-prefill shape with
fp8 and fp4 operands and the fused epilogue, the decode shape in GB/s with
weights rotated through more copies than the 256 MB MALL holds, the
quantizer, the dequantize-to-fp16 ablation), the MFMA ceiling on each
workload's own operand bytes, the observed shader clock, and the CPU oracle
on every configuration.

Timing protocol (the published-peak fractions use it): warm-up of at least
20 launches and 60 ms of GPU time (past the power transient that follows
any idle gap), then 7 windows of back-to-back launches of at least 2 ms each between HIP
events recorded on the stream the kernels are launched on; the median and
the minimum of the per-launch times over the windows are reported (short
kernels are replayed from a captured HIP graph so that the GPU, not the
Python call rate, is timed).  The shader clock under the GEMM's MFMA load is
read inside the MFMA-ceiling kernel (s_memtime cycles against the 100 MHz
s_memrealtime ticks of each workgroup's first wave).  The contract's own
measurement (W warm-up launches, then exactly K timed launches) runs after
the windows, on a warm GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import struct
import subprocess
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 GEMM TFLOP/s (% of fp8 peak) at 8192³; fp8/fp16 ratio; decode GB/s"
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 MFMA
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4 MFMA
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
LIB = os.path.join(ROOT, "block_scaled_precision_mxgemm_amd", "libmxgemm.so")
LLVM_BIN = "/opt/rocm/llvm/bin"
WINDOWS = 7
WINDOW_MS = 2.0
WARMUP = 20
# After an idle gap the GPU runs a power transient: the first launches of a
# large GEMM are fast, the next ones up to 30 % slower, and the rate settles
# after ~25 ms of continuous work (measured).  Every measurement therefore
# warms up for at least this long as well as for WARMUP launches.
WARM_MS = 60.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ provenance

def _sha16_files(paths):
    h = hashlib.sha256()
    for p in sorted(paths):
        h.update(os.path.relpath(p, ROOT).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def provenance(dev_props):
    """Commit (when the tree is a git checkout), digests of the sources, the
    built library and the environment: enough to tell which build and which
    software stack produced a number."""
    import torch

    pkg = os.path.join(ROOT, "block_scaled_precision_mxgemm_amd")
    srcs = [os.path.join(pkg, "csrc", f) for f in os.listdir(os.path.join(pkg, "csrc"))]
    srcs += [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    srcs += [os.path.join(pkg, f) for f in ("mxgemm.py", "inputs.py")] + [os.path.abspath(__file__)]
    head = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            head = r.stdout.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    env = {
        "python": platform.python_version(),
        "torch": torch.__version__,
        "hip": getattr(torch.version, "hip", None),
        "device": dev_props.name,
        "arch": dev_props.gcnArchName,
        "cus": dev_props.multi_processor_count,
        "hbm_bytes": dev_props.total_memory,
        "host_cpus": os.cpu_count(),
    }
    try:
        with open("/sys/module/amdgpu/version") as f:
            env["amdgpu_driver"] = f.read().strip()
    except OSError:
        pass
    return {
        "git_head": head,
        "source_digest": _sha16_files(srcs),
        "library_digest": _sha16_files([LIB]) if os.path.exists(LIB) else None,
        "env": env,
        "env_digest": hashlib.sha256(json.dumps(env, sort_keys=True).encode()).hexdigest()[:16],
        "inputs": "block_scaled_precision_mxgemm_amd/inputs.py recipes, numpy PCG64 seeds per workload",
    }


# ---------------------------------------------------------------------- timing

def time_steps(fn, steps: int, warmup: int):
    """The contract's timing: `warmup` untimed launches, then exactly `steps`
    launches between two events on the launch stream, synchronized on both
    sides.  Returns milliseconds per launch.  Before the warm-up launches the
    GPU is kept busy with fn for WARM_MS (untimed), so the timed launches do
    not fall into the power transient that follows any idle gap of a few ms
    (host work between measurements is one)."""
    import torch

    warm_gpu(fn, 0)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for i in range(steps):
        fn(i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def warm_gpu(fn, launches: int, warm_ms=None):
    """At least `launches` launches of fn and at least warm_ms (default
    WARM_MS) of its GPU time, back to back, then a synchronize."""
    import torch

    warm_ms = WARM_MS if warm_ms is None else warm_ms
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    fn(0)
    e1.record(s)
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    n = max(launches - 1, int(math.ceil(warm_ms / one)) if warm_ms > 0 else 0)
    for i in range(min(n, 100000)):
        fn(i + 1)
    torch.cuda.synchronize()


def time_windows(fn, warmup=None, windows=None, min_ms=None):
    """Warm-up (`warmup` launches, default 20, lasting at least WARM_MS of GPU
    time), then `windows` (7) windows of R
    back-to-back launches (R chosen so a window lasts >= min_ms, 2 ms) with an
    event between windows.  Returns median / min / max milliseconds per launch
    over the windows."""
    import torch

    warmup = WARMUP if warmup is None else warmup
    windows = WINDOWS if windows is None else windows
    min_ms = WINDOW_MS if min_ms is None else min_ms
    warm_gpu(fn, warmup)
    s = torch.cuda.current_stream()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(s)
    for i in range(3):
        fn(i)
    c1.record(s)
    torch.cuda.synchronize()
    one = max(c0.elapsed_time(c1) / 3, 1e-4)
    R = max(1, int(math.ceil(min_ms * 1.1 / one)))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(windows + 1)]
    ev[0].record(s)
    n = 0
    for w in range(windows):
        for _ in range(R):
            fn(n)
            n += 1
        ev[w + 1].record(s)
    torch.cuda.synchronize()
    per = np.array([ev[w].elapsed_time(ev[w + 1]) / R for w in range(windows)])
    return {"ms_median": float(np.median(per)), "ms_min": float(per.min()), "ms_max": float(per.max()),
            "windows": windows, "launches_per_window": R, "window_ms_median": float(np.median(per) * R)}


def time_graph_windows(fn, launches: int, warmup=None, windows=None, min_ms=None):
    """As time_windows, with the launches replayed from a captured HIP graph of
    `launches` calls (no host work between kernels)."""
    import torch

    warmup = WARMUP if warmup is None else warmup
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(launches):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    res = time_windows(lambda i=0: g.replay(), warmup=2, windows=windows, min_ms=min_ms)
    torch.cuda.synchronize()
    del g
    for k in ("ms_median", "ms_min", "ms_max"):
        res[k] /= launches
    res["graph_launches"] = launches
    return res


def tflops(flops, ms):
    return flops / (ms * 1e-3) / 1e12


def timed_entry(res, flops=None, nbytes=None, peak=None, peak_unit="TFLOP/s"):
    """A workload record: median timing and the derived rate(s)."""
    ms = res["ms_median"]
    out = {"ms": ms, "ms_min": res["ms_min"], "ms_max": res["ms_max"],
           "timing": "median of %d windows x %d launches%s" % (res["windows"], res["launches_per_window"],
                                                              " (graph of %d)" % res["graph_launches"]
                                                              if "graph_launches" in res else "")}
    if flops is not None:
        out["TFLOP/s"] = tflops(flops, ms)
        out["TFLOP/s_best"] = tflops(flops, res["ms_min"])
        if peak is not None and peak_unit == "TFLOP/s":
            out["peak_frac"] = out["TFLOP/s"] / peak
    if nbytes is not None:
        out["GB/s"] = nbytes / (ms * 1e-3) / 1e9
        out["hbm_frac"] = out["GB/s"] / PEAK_HBM_GBPS
    return out


# ------------------------------------------------------- kernel code digest

def _code_objects(lib_path):
    """gfx950 code objects bundled in the library's .hip_fatbin section."""
    with tempfile.TemporaryDirectory() as d:
        fb = os.path.join(d, "fatbin")
        subprocess.run([os.path.join(LLVM_BIN, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fb, lib_path,
                        os.path.join(d, "stripped")], check=True, capture_output=True)
        data = open(fb, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    pos, cos = 0, []
    while True:
        i = data.find(magic, pos)
        if i < 0:
            break
        (n,) = struct.unpack_from("<Q", data, i + 24)
        off = i + 32
        for _ in range(n):
            o, sz, tl = struct.unpack_from("<QQQ", data, off)
            off += 24
            triple = data[off:off + tl].decode()
            off += tl
            if "gfx950" in triple:
                cos.append(data[i + o:i + o + sz])
        pos = i + 1
    return cos


def kernel_code_digest(symbol_prefix: str, lib_path: str = LIB):
    """sha256 (16 hex) of the disassembled instructions of the first kernel
    whose mangled name contains `symbol_prefix`, from the built library (branch
    offsets are relative, so moving other kernels does not change it).  None if
    the tools or the kernel are missing."""
    try:
        with tempfile.TemporaryDirectory() as d:
            for k, co in enumerate(_code_objects(lib_path)):
                p = os.path.join(d, "co%d" % k)
                with open(p, "wb") as f:
                    f.write(co)
                syms = subprocess.run([os.path.join(LLVM_BIN, "llvm-readelf"), "--symbols", "--wide", p],
                                      capture_output=True, text=True, check=True).stdout
                names = [ln.split()[-1] for ln in syms.splitlines() if " FUNC " in ln and symbol_prefix in ln]
                if not names:
                    continue
                dis = subprocess.run([os.path.join(LLVM_BIN, "llvm-objdump"), "-d", "--no-show-raw-insn",
                                      "--no-leading-addr", "--disassemble-symbols=" + names[0], p],
                                     capture_output=True, text=True, check=True).stdout
                body = [ln.split("//")[0].strip() for ln in dis.splitlines() if ln.startswith("\t")]
                h = hashlib.sha256(("\n".join(x for x in body if x)).encode()).hexdigest()[:16]
                return {"symbol": names[0], "code_digest": h}
    except (OSError, subprocess.SubprocessError, ValueError):
        return None
    return None


def traffic_entry(entry: str):
    """HBM bytes per launch of one workload's kernel from the committed
    rocprofv3 counter runs, if they were taken on the kernel code that the
    current library holds (same disassembly digest); else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("entries", {}).get(entry)
    if not e:
        return None
    cur = kernel_code_digest(e.get("symbol", "\0"))
    if cur is None or cur["code_digest"] != e.get("code_digest"):
        return None
    return e.get("bytes_per_launch")


# ------------------------------------------------------------ MFMA ceiling

def mfma_ceiling(mx, ops, scales, kind, ms_target=4.0):
    """Median TFLOP/s of the ceiling kernel on the given operand bytes (one
    workgroup of 8 waves per CU, iterations sized to ~ms_target per launch),
    and the shader clock its waves measured (median over workgroups of one
    launch, s_memtime cycles / s_memrealtime ticks x 100 MHz)."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float32, device=ops.device)
    clocks = torch.zeros(cus * 2, dtype=torch.int32, device=ops.device)
    probe_iters = 256
    # per wave and round: 32 scaled 16x16x128 MFMAs, or 64 fp16 16x16x32 ones
    flops_per_iter = cus * 8 * (64 * 16384 if kind == mx.CEIL_FP16 else 32 * 65536)
    r0 = time_windows(lambda i=0: mx.mxgemm_mfma_ceiling(ops, scales, kind, probe_iters, cus, out=out), warmup=3,
                      windows=3, min_ms=0.5)
    rate = flops_per_iter * probe_iters / (r0["ms_median"] * 1e-3)
    iters = int(max(64, min(1 << 20, rate * ms_target * 1e-3 / flops_per_iter)))
    run = lambda i=0: mx.mxgemm_mfma_ceiling(ops, scales, kind, iters, cus, out=out)
    r = time_windows(run, warmup=3)
    mx.mxgemm_mfma_ceiling(ops, scales, kind, iters, cus, out=out, clocks=clocks)
    ck = clocks.view(cus, 2).cpu().numpy().astype(np.float64)
    ok = ck[:, 1] > 0
    mhz = ck[ok, 0] / ck[ok, 1] * 100.0
    return {"TFLOP/s": tflops(flops_per_iter * iters, r["ms_median"]),
            "TFLOP/s_best": tflops(flops_per_iter * iters, r["ms_min"]), "ms": r["ms_median"], "iters": iters,
            "workgroups": cus,
            "sclk_mhz": float(np.median(mhz)) if mhz.size else None,
            "sclk_mhz_range": [float(mhz.min()), float(mhz.max())] if mhz.size else None}


# ------------------------------------------------------------ CPU baseline

def _oracle_time(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def cpu_baselines(full: bool, budget_s: float):
    """Time the oracle (as it stands) on every configuration, on the host
    cores: all threads, and one thread on the three small configurations.
    Configurations too large for the budget are timed on a seeded sample of
    output elements (every sampled element is a full-K float64 dot product);
    `full` runs everything in full.  Returns (headline record, all records)."""
    import oracle
    from block_scaled_precision_mxgemm_amd import inputs as mxin

    nthreads = oracle.num_threads()
    recs = {}
    cache = {}

    def mx_ops(w, ea, eb):
        # the workload's operands quantized by the oracle itself
        if w.name not in cache:
            cache.clear()
            a32, b32 = mxin.mx_sources(w)
            qa, sa = oracle.quantize(a32, ea)
            qb, sb = oracle.quantize(b32, eb)
            cache[w.name] = (qa, sa, qb, sb)
        return cache[w.name]

    def run_mx(name, ea, eb, threads, rows=None, npts=None, seed=11):
        w = mxin.WORKLOADS[name]
        qa, sa, qb, sb = mx_ops(w, ea, eb)
        oracle.set_num_threads(threads)
        if npts is not None:
            rng = np.random.default_rng(seed)
            I = rng.integers(0, w.M, npts)
            J = rng.integers(0, w.N, npts)
            dt = _oracle_time(lambda: oracle.mx_gemm(qa, sa, ea, qb, sb, eb, w.M, w.N, w.K, points=(I, J)))
            flops, what = 2.0 * w.K * npts, "%d random output elements (seed %d)" % (npts, seed)
        elif rows is not None and rows < w.M:
            dt = _oracle_time(lambda: oracle.mx_gemm(qa[:rows], sa[:rows], ea, qb, sb, eb, rows, w.N, w.K))
            flops, what = 2.0 * rows * w.N * w.K, "the first %d of %d rows (every column)" % (rows, w.M)
        else:
            dt = _oracle_time(lambda: oracle.mx_gemm(qa, sa, ea, qb, sb, eb, w.M, w.N, w.K))
            flops, what = 2.0 * w.M * w.N * w.K, "full"
        oracle.set_num_threads(nthreads)
        return {"GFLOP/s": flops / dt / 1e9, "seconds": dt, "threads": threads, "work": what}

    def run_f16(name, b_is_nk, threads, rows=None):
        w = mxin.WORKLOADS[name]
        a16, b16 = mxin.fp16_sources(w, b_is_nk=b_is_nk)
        M = w.M if rows is None else rows
        oracle.set_num_threads(threads)
        dt = _oracle_time(lambda: oracle.fp16_gemm(a16[:M].view(np.uint16), b16.view(np.uint16), M, w.N, w.K,
                                                   int(b_is_nk)))
        oracle.set_num_threads(nthreads)
        what = "full" if M == w.M else "the first %d of %d rows (every column)" % (M, w.M)
        return {"GFLOP/s": 2.0 * M * w.N * w.K / dt / 1e9, "seconds": dt, "threads": threads, "work": what}

    E4, E2 = oracle.E4M3, oracle.E2M1
    recs["mxfp8_256"] = {"all_threads": run_mx("mxfp8_256", E4, E4, nthreads),
                         "one_thread": run_mx("mxfp8_256", E4, E4, 1)}
    recs["fp16_1024"] = {"all_threads": run_f16("fp16_1024", False, nthreads),
                         "one_thread": run_f16("fp16_1024", False, 1, rows=None if full else 64)}
    recs["mxfp8_2048"] = {"all_threads": run_mx("mxfp8_2048", E4, E4, nthreads),
                          "one_thread": run_mx("mxfp8_2048", E4, E4, 1, rows=None if full else 128)}
    recs["decode_16x28672x8192"] = {"all_threads": run_mx("decode_16x28672x8192", E4, E2, nthreads)}
    # the two large products: a sample sized to the budget unless full
    big = {}
    for name in ("prefill_8192x14336x4096", "mxfp8_8192"):
        w = mxin.WORKLOADS[name]
        if full:
            big[name] = run_mx(name, E4, E4, nthreads)
            continue
        probe = run_mx(name, E4, E4, nthreads, npts=20000, seed=10)
        rate_pts = 20000 / probe["seconds"]
        npts = int(max(20000, min(16_000_000, rate_pts * budget_s / 2)))
        big[name] = run_mx(name, E4, E4, nthreads, npts=npts)
    recs["prefill_8192x14336x4096"] = {"all_threads": big["prefill_8192x14336x4096"]}
    recs["mxfp8_8192"] = {"all_threads": big["mxfp8_8192"]}
    h = big["mxfp8_8192"]
    headline = {
        "value": h["GFLOP/s"] / 1e3,
        "unit": "TFLOP/s",
        "cores": nthreads,
        "kind": "oracle",
        "sample": "%s of the 8192x8192x8192 MXFP8 product (each a full K=8192 float64 dot product over E4M3 codes "
                  "and UE8M0 scales decoded by table), %.1f s wall on %d threads" % (h["work"], h["seconds"], nthreads),
        "gflops": h["GFLOP/s"],
    }
    return headline, recs


# ------------------------------------------------------------------ workloads

def mx_operands(name, dev):
    """The workload's fp32 sources on the device and their MX codes and
    scales (quantized on the GPU), in the workload's element formats."""
    import torch

    from block_scaled_precision_mxgemm_amd import inputs as mxin
    from block_scaled_precision_mxgemm_amd import mxgemm as mx

    w = mxin.WORKLOADS[name]
    a32, b32 = mxin.mx_sources(w)
    ta = torch.from_numpy(a32).to(dev)
    tb = torch.from_numpy(b32).to(dev)
    del a32, b32
    elem = {"e4m3": mx.E4M3, "e5m2": mx.E5M2, "e2m1": mx.E2M1, "int4": mx.INT4, "int2": mx.INT2,
            "e2m3": mx.E2M3, "e3m2": mx.E3M2}
    qa, sa = mx.mxgemm_quantize(ta, elem[w.elem_a])
    qb, sb = mx.mxgemm_quantize(tb, elem[w.elem_b])
    torch.cuda.synchronize()
    return w, ta, tb, qa, sa, qb, sb


def bench_decode(dev, name="decode_16x28672x8192"):
    """MXFP8 activations x the workload's weights (E2M1, INT4 or INT2),
    16 x 28672 x 8192, weights rotated over copies larger in total than the
    MALL so every launch reads HBM."""
    import torch

    from block_scaled_precision_mxgemm_amd import inputs as mxin
    from block_scaled_precision_mxgemm_amd import mxgemm as mx

    w = mxin.WORKLOADS[name]
    elem, fmt, kname = {"e2m1": (mx.E2M1, mx.FMT_FP8_FP4, "fp4"), "int4": (mx.INT4, mx.FMT_FP8_INT4, "int4"),
                        "int2": (mx.INT2, mx.FMT_FP8_INT2, "int2"), "e2m3": (mx.E2M3, mx.FMT_FP8_FP6, "e2m3"),
                        "e3m2": (mx.E3M2, mx.FMT_FP8_BF6, "e3m2")}[w.elem_b]
    a32, _ = mxin.mx_sources(w, N=1)
    qa, sa = mx.mxgemm_quantize(torch.from_numpy(a32).to(dev), mx.E4M3)
    wb = w.N * w.K * {mx.INT2: 1, mx.E2M3: 3, mx.E3M2: 3}.get(elem, 2) // 4   # weight bytes
    copies = max(5, int(math.ceil(600e6 / (wb + w.N * w.K // 32))))   # > 2x the 256 MB MALL in total
    weights = []
    for b32 in mxin.decode_weight_copies(w, copies):
        tb = torch.from_numpy(b32).to(dev)
        del b32
        weights.append(mx.mxgemm_quantize(tb, elem))
        del tb
    torch.cuda.synchronize()
    c = torch.empty((w.M, w.N), dtype=torch.float32, device=dev)
    nbytes = (w.M * w.K + w.M * w.K // 32 + wb + w.N * w.K // 32 + w.M * w.N * 4)
    step = lambda i=0: mx.mxgemm_run(qa, sa, weights[i % copies][0], weights[i % copies][1], fmt, out=c)
    # A decode step runs inside a serving loop, as a captured graph: the
    # primary figure replays a graph of 8 rounds over the weight copies (no
    # host launch gap between kernels); the eager figure (one host launch per
    # kernel, ~1 us gap each) is kept beside it.
    cold = time_graph_windows(step, 8 * copies)
    eager = time_windows(step)
    warm = time_windows(lambda i=0: mx.mxgemm_run(qa, sa, weights[0][0], weights[0][1], fmt, out=c))
    rec = timed_entry(cold, nbytes=nbytes)
    kernel = "decode_kernel<fp8 x %s, K=8192> (LDS-staged weight stream)" % kname
    rec.update({"kernel": kernel,
                "us": rec["ms"] * 1e3, "us_best": rec["ms_min"] * 1e3, "algorithmic_bytes": nbytes,
                "weight_copies_rotated": copies,
                "eager_us": eager["ms_median"] * 1e3, "eager_GB/s": nbytes / (eager["ms_median"] * 1e-3) / 1e9,
                "eager_hbm_frac": nbytes / (eager["ms_median"] * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "warm_us_mall_resident": warm["ms_median"] * 1e3,
                "warm_GB/s": nbytes / (warm["ms_median"] * 1e-3) / 1e9})
    if name == "decode_16x28672x8192":
        rec["traffic"] = traffic_entry("decode_16x28672x8192")
    log("%s: cold %.2f us graph-replayed (%.0f GB/s, %.1f%% of HBM), %.2f us eager, warm %.2f us" % (
        name, rec["us"], rec["GB/s"], 100 * rec["hbm_frac"], rec["eager_us"], warm["ms_median"] * 1e3))
    return rec


def main():
    global WINDOWS, WINDOW_MS, WARMUP, WARM_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["all", "headline", "decode", "int", "fp6", "fp16", "prefill", "small",
                                       "ceiling"],
                    default="all", help="run a subset (for profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle time budget for each of the two sampled large configurations")
    ap.add_argument("--cpu-full", action="store_true", help="run the oracle in full on every configuration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--windows", type=int, default=WINDOWS, help="timing windows per measurement")
    ap.add_argument("--window-ms", type=float, default=WINDOW_MS, help="least duration of one window")
    ap.add_argument("--window-warmup", type=int, default=WARMUP, help="warm-up launches before the windows")
    ap.add_argument("--warm-ms", type=float, default=WARM_MS, help="least GPU time of every warm-up")
    args = ap.parse_args()
    WINDOWS, WINDOW_MS, WARMUP = max(1, args.windows), max(0.0, args.window_ms), max(0, args.window_warmup)
    WARM_MS = max(0.0, args.warm_ms)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_scaled_precision_mxgemm_amd import inputs as mxin
    from block_scaled_precision_mxgemm_amd import mxgemm as mx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if not mx.mxgemm_device_supported():
        raise SystemExit("device is not gfx950")
    props = torch.cuda.get_device_properties(0)
    extra = {}
    ceilings = {}
    only = args.only

    # ---------------- headline: MXFP8 8192^3 ---------------------------------
    log("headline: generating and quantizing 8192^3 operands")
    w, ta, tb, qa, sa, qb, sb = mx_operands("mxfp8_8192", dev)
    M, N, K = w.M, w.N, w.K
    c = torch.empty((M, N), dtype=torch.float32, device=dev)
    flops = 2.0 * M * N * K
    run8 = lambda i=0: mx.mxgemm_run(qa, sa, qb, sb, mx.FMT_FP8_FP8, out=c)
    warm_gpu(run8, 0, warm_ms=2 * WARM_MS)   # past the power transient before anything is timed
    head_w = time_windows(run8)
    ms = time_steps(run8, args.steps, args.warmup)
    log("mxfp8 8192^3: windows median %.4f ms, min %.4f ms; %.4f ms over the %d contract steps (%.1f TFLOP/s)" % (
        head_w["ms_median"], head_w["ms_min"], ms, args.steps, tflops(flops, ms)))
    extra["mxfp8_8192_windows"] = timed_entry(head_w, flops=flops, peak=PEAK_FP8_TFLOPS)

    if only in ("all", "headline", "ceiling"):
        ceilings["fp8_e4m3"] = mfma_ceiling(mx, qa, sa, mx.FMT_FP8_FP8)
        log("MFMA ceiling fp8 on the 8192^3 operands: %.0f TFLOP/s at %s MHz" % (
            ceilings["fp8_e4m3"]["TFLOP/s"], ceilings["fp8_e4m3"]["sclk_mhz"]))
    if only in ("all", "headline"):
        # The inputs are rotated over three 256 MiB copies (more than twice the
        # 256 MB MALL in total), so every launch reads its input from HBM; the
        # figure with one input, part of which stays in the MALL between
        # launches, is kept beside it.
        xs = [ta, tb, torch.randn_like(ta)]
        qb4 = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        sb4 = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
        for name, elem, q_, s_, per_el in (("quantize_8192x8192_e4m3", mx.E4M3, qa, sa, 4 + 1 + 1 / 32),
                                           ("quantize_8192x8192_e2m1", mx.E2M1, qb4, sb4, 4 + 0.5 + 1 / 32)):
            nbytes = M * K * per_el
            cold = time_windows(lambda i=0: mx.mxgemm_quantize(xs[i % len(xs)], elem, q=q_, s=s_))
            warm = time_windows(lambda i=0: mx.mxgemm_quantize(ta, elem, q=q_, s=s_))
            rec = timed_entry(cold, nbytes=nbytes)
            rec.update({"inputs_rotated": len(xs), "one_input_us": warm["ms_median"] * 1e3,
                        "one_input_GB/s": nbytes / (warm["ms_median"] * 1e-3) / 1e9})
            extra[name] = rec
            log("%s: %.1f us = %.0f GB/s (%.1f%% of HBM) with inputs from HBM; %.1f us with one input" % (
                name, cold["ms_median"] * 1e3, rec["GB/s"], 100 * rec["hbm_frac"], warm["ms_median"] * 1e3))
        # the E4M3 runs leave in qa / sa the codes of whichever input came
        # last: restore the headline operands
        mx.mxgemm_quantize(ta, mx.E4M3, q=qa, s=sa)
        del xs
        del qb4, sb4
    if only == "all":
        # E4M3 activations x E5M2 weights on the same sources
        qb5, sb5 = mx.mxgemm_quantize(tb, mx.E5M2)
        r45 = time_windows(lambda i=0: mx.mxgemm_run(qa, sa, qb5, sb5, mx.FMT_FP8_BF8, out=c))
        extra["mxfp8xbf8_8192"] = timed_entry(r45, flops=flops, peak=PEAK_FP8_TFLOPS)
        del qb5, sb5
    del ta, tb

    if only in ("all", "fp16"):
        a16, b16 = mxin.fp16_sources(w, b_is_nk=True)
        ta16 = torch.from_numpy(a16).to(dev)
        tb16 = torch.from_numpy(b16).to(dev)
        del a16, b16
        f8 = time_windows(lambda i=0: mx.fp16gemm_run(ta16, tb16, True, out=c))
        extra["fp16_8192"] = timed_entry(f8, flops=flops, peak=PEAK_FP16_TFLOPS)
        ratio = f8["ms_median"] / head_w["ms_median"]
        extra["fp8_fp16_ratio_8192"] = ratio
        extra["fp8_verdict_8192"] = "accelerated" if ratio >= 1.5 else "emulated"
        ceilings["fp16"] = mfma_ceiling(mx, ta16.view(torch.uint8), None, mx.CEIL_FP16)
        log("fp16 8192^3: %.3f ms, ratio %.2f; MFMA ceiling fp16 %.0f TFLOP/s" % (
            f8["ms_median"], ratio, ceilings["fp16"]["TFLOP/s"]))
        del ta16, tb16

    if only == "all":
        c16 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        rb = time_windows(lambda i=0: mx.mxgemm_run_fused(qa, sa, qb, sb, mx.FMT_FP8_FP8, out_type=mx.OUT_BF16,
                                                           out=c16))
        extra["mxfp8_8192_bf16_out"] = timed_entry(rb, flops=flops, peak=PEAK_FP8_TFLOPS)
        del c16
        rd = time_windows(lambda i=0: mx.mxgemm_run_dequant_fp16(qa, sa, qb, sb, mx.FMT_FP8_FP8, out=c), warmup=3)
        extra["ablation_dequant_fp16_8192"] = timed_entry(rd, flops=flops)
        extra["ablation_dequant_fp16_8192"]["scaled_mfma_speedup"] = rd["ms_median"] / head_w["ms_median"]

    del c, qa, sa, qb, sb
    torch.cuda.empty_cache()

    if only in ("all", "small"):
        # 2048^3 pair (the RIGEL ratio point) ---------------------------------
        w3, ta, tb, qa3, sa3, qb3, sb3 = mx_operands("mxfp8_2048", dev)
        c3 = torch.empty((w3.M, w3.N), dtype=torch.float32, device=dev)
        f3 = 2.0 * w3.M * w3.N * w3.K
        run3 = lambda i=0: mx.mxgemm_run(qa3, sa3, qb3, sb3, 0, out=c3)
        r3 = time_graph_windows(run3, 50)
        a16, b16 = mxin.fp16_sources(w3, b_is_nk=True)
        ta16, tb16 = torch.from_numpy(a16).to(dev), torch.from_numpy(b16).to(dev)
        rf3 = time_graph_windows(lambda i=0: mx.fp16gemm_run(ta16, tb16, True, out=c3), 50)
        extra["mxfp8_2048"] = timed_entry(r3, flops=f3, peak=PEAK_FP8_TFLOPS)
        extra["fp16_2048"] = timed_entry(rf3, flops=f3, peak=PEAK_FP16_TFLOPS)
        extra["fp8_fp16_ratio_2048"] = rf3["ms_median"] / r3["ms_median"]
        extra["fp8_verdict_2048"] = "accelerated" if extra["fp8_fp16_ratio_2048"] >= 1.5 else "emulated"
        rd3 = time_graph_windows(lambda i=0: mx.mxgemm_run_dequant_fp16(qa3, sa3, qb3, sb3, 0, out=c3), 10)
        extra["ablation_dequant_fp16_2048"] = timed_entry(rd3, flops=f3)
        extra["ablation_dequant_fp16_2048"]["scaled_mfma_speedup"] = rd3["ms_median"] / r3["ms_median"]
        del ta, tb, qa3, sa3, qb3, sb3, ta16, tb16, c3

        # fp16 1024^3, row-major A and B ---------------------------------------
        w2 = mxin.WORKLOADS["fp16_1024"]
        a16, b16 = mxin.fp16_sources(w2, b_is_nk=False)
        ta16, tb16 = torch.from_numpy(a16).to(dev), torch.from_numpy(b16).to(dev)
        c2 = torch.empty((w2.M, w2.N), dtype=torch.float32, device=dev)
        r2 = time_graph_windows(lambda i=0: mx.fp16gemm_run(ta16, tb16, False, out=c2), 100)
        extra["fp16_1024_kn"] = timed_entry(r2, flops=2.0 * 1024 ** 3, peak=PEAK_FP16_TFLOPS)
        del ta16, tb16, c2

        # MXFP8 256^3 -----------------------------------------------------------
        w1, ta, tb, qa1, sa1, qb1, sb1 = mx_operands("mxfp8_256", dev)
        c1 = torch.empty((256, 256), dtype=torch.float32, device=dev)
        r1 = time_graph_windows(lambda i=0: mx.mxgemm_run(qa1, sa1, qb1, sb1, 0, out=c1), 200)
        extra["mxfp8_256"] = timed_entry(r1, flops=2.0 * 256 ** 3, peak=PEAK_FP8_TFLOPS)
        extra["mxfp8_256"]["note"] = "4 workgroups (128x128 tiles) on 256 CUs: latency bound"
        del ta, tb, qa1, sa1, qb1, sb1, c1

    if only in ("all", "prefill"):
        # LLM prefill 8192 x 14336 x 4096 --------------------------------------
        w4, ta, tb, qa4, sa4, qb4, sb4 = mx_operands("prefill_8192x14336x4096", dev)
        del ta, tb
        c4 = torch.empty((w4.M, w4.N), dtype=torch.float32, device=dev)
        f4 = 2.0 * w4.M * w4.N * w4.K
        r4 = time_windows(lambda i=0: mx.mxgemm_run(qa4, sa4, qb4, sb4, 0, out=c4))
        extra["prefill_8192x14336x4096"] = timed_entry(r4, flops=f4, peak=PEAK_FP8_TFLOPS)
        bias4 = torch.from_numpy(np.random.default_rng(44).standard_normal(w4.N).astype(np.float32)).to(dev)
        c16 = torch.empty((w4.M, w4.N), dtype=torch.bfloat16, device=dev)
        fz = lambda i=0: mx.mxgemm_run_fused(qa4, sa4, qb4, sb4, 0, bias=bias4, act=mx.ACT_GELU,
                                             out_type=mx.OUT_BF16, out=c16)
        rz = time_windows(fz)
        ep = lambda i=0: mx.mxgemm_epilogue(c4, bias4, mx.ACT_GELU, mx.OUT_BF16, out=c16)
        rep = time_windows(ep)
        rdz = time_windows(lambda i=0: (mx.mxgemm_run(qa4, sa4, qb4, sb4, 0, out=c4), ep()))
        ep_bytes = w4.M * w4.N * (4 + 2) + w4.N * 4
        fused = timed_entry(rz, flops=f4, peak=PEAK_FP8_TFLOPS)
        fused.update({"decomposed_ms": rdz["ms_median"], "fused_speedup": rdz["ms_median"] / rz["ms_median"],
                      "epilogue_pass_ms": rep["ms_median"],
                      "epilogue_pass_GB/s": ep_bytes / (rep["ms_median"] * 1e-3) / 1e9,
                      "note": "C = bf16(GELU(A B^T + bias)); decomposed = fp32 GEMM + separate epilogue pass"})
        extra["prefill_fused_bias_gelu_bf16"] = fused
        rd4 = time_windows(lambda i=0: mx.mxgemm_run_dequant_fp16(qa4, sa4, qb4, sb4, 0, out=c4), warmup=3)
        extra["ablation_dequant_fp16_prefill"] = timed_entry(rd4, flops=f4)
        extra["ablation_dequant_fp16_prefill"]["scaled_mfma_speedup"] = rd4["ms_median"] / r4["ms_median"]
        del qa4, sa4, qb4, sb4, c16

        # the same prefill GEMM with both operands MXFP4 (E2M1), against the fp4 roof
        w5, ta, tb, qa5, sa5, qb5, sb5 = mx_operands("prefill_mxfp4_8192x14336x4096", dev)
        del ta, tb
        r5 = time_windows(lambda i=0: mx.mxgemm_run(qa5, sa5, qb5, sb5, mx.FMT_FP4_FP4, out=c4))
        extra["prefill_mxfp4_8192x14336x4096"] = timed_entry(r5, flops=f4, peak=PEAK_FP4_TFLOPS)
        ceilings["fp4_e2m1"] = mfma_ceiling(mx, qa5, sa5, mx.FMT_FP4_FP4)
        extra["prefill_mxfp4_8192x14336x4096"]["ceiling_frac"] = (
            extra["prefill_mxfp4_8192x14336x4096"]["TFLOP/s"] / ceilings["fp4_e2m1"]["TFLOP/s"])
        del qa5, sa5, qb5, sb5

        # the same prefill GEMM with E4M3 activations and FP6 / INT4 / INT2
        # weights (the 4-wave tiled kernel), against the fp8 peak: one MFMA
        # operand is E4M3 (INT4 runs E4M3 x E4M3, INT2 E4M3 x E2M1 after the
        # remap); the E4M3 x E2M1 MFMA ceiling is measured beside it
        for name, fmt in (("prefill_e2m3_8192x14336x4096", mx.FMT_FP8_FP6),
                          ("prefill_int4_8192x14336x4096", mx.FMT_FP8_INT4),
                          ("prefill_int2_8192x14336x4096", mx.FMT_FP8_INT2)):
            wq, ta, tb, qaq, saq, qbq, sbq = mx_operands(name, dev)
            del ta, tb
            rq = time_windows(lambda i=0: mx.mxgemm_run(qaq, saq, qbq, sbq, fmt, out=c4))
            extra[name] = timed_entry(rq, flops=f4, peak=PEAK_FP8_TFLOPS)
            log("%s: %.3f ms = %.0f TFLOP/s (%.1f%% of the fp8 peak)" % (
                name, rq["ms_median"], extra[name]["TFLOP/s"], 100 * extra[name]["peak_frac"]))
            if fmt == mx.FMT_FP8_INT2:
                ceilings["fp8_e2m1"] = mfma_ceiling(mx, qaq, saq, mx.FMT_FP8_FP4)
                log("MFMA ceiling E4M3 x E2M1: %.0f TFLOP/s" % ceilings["fp8_e2m1"]["TFLOP/s"])
                extra[name]["ceiling_frac"] = extra[name]["TFLOP/s"] / ceilings["fp8_e2m1"]["TFLOP/s"]
            del qaq, saq, qbq, sbq
        del c4
        torch.cuda.empty_cache()

    if only in ("all", "decode"):
        extra["decode_16x28672x8192"] = bench_decode(dev)
    if only in ("all", "decode", "int"):
        for name in ("decode_int4_16x28672x8192", "decode_int2_16x28672x8192"):
            extra[name] = bench_decode(dev, name)
    if only in ("all", "decode", "fp6"):
        for name in ("decode_e2m3_16x28672x8192", "decode_e3m2_16x28672x8192"):
            extra[name] = bench_decode(dev, name)

    cpu = None
    if not args.no_cpu_baseline and only == "all":
        log("cpu baseline: timing the oracle on every configuration")
        cpu, cpu_all = cpu_baselines(args.cpu_full, args.cpu_seconds)
        extra["cpu_baseline_configs"] = cpu_all

    value = tflops(flops, ms)
    achieved = tflops(flops, head_w["ms_median"])
    code = kernel_code_digest("pingpong_kernelINS0_5PPCfgILi0ELi0ELi0E")
    roof = {
        "bound": "mfma",
        "achieved": achieved,
        "peak": PEAK_FP8_TFLOPS,
        "unit": "TFLOP/s",
        "frac": achieved / PEAK_FP8_TFLOPS,
        "traffic": traffic_entry("mx_gemm_8192"),
        "kernel": "pingpong_kernel<MX fp8 x fp8, 256x256, 8 waves>",
        "kernel_code_digest": code["code_digest"] if code else None,
        "achieved_timing": "median of %d windows of %d launches (HIP events on the launch stream), after %d warm-up"
                           % (head_w["windows"], head_w["launches_per_window"], WARMUP),
        "achieved_best": tflops(flops, head_w["ms_min"]),
    }
    if "fp8_e4m3" in ceilings:
        roof["measured_ceiling"] = ceilings["fp8_e4m3"]["TFLOP/s"]
        roof["ceiling_frac"] = achieved / ceilings["fp8_e4m3"]["TFLOP/s"]
        mhz = ceilings["fp8_e4m3"].get("sclk_mhz")
        if mhz:
            roof["sclk_mhz_under_mfma_load"] = mhz
            roof["clock_adjusted_peak"] = PEAK_FP8_TFLOPS * mhz / 2400.0
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (UE8M0 per 32 K), fp32 accumulate",
        "data": "synthetic (seeded numpy PCG64, N(0,1) operands)",
        "config": {"workload": "mxfp8_8192", "M": M, "N": N, "K": K, "fmt": "E4M3 x E4M3",
                   "scale": "UE8M0 per 32 K", "out": "fp32"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "mfma_ceiling": ceilings,
        "provenance": provenance(props),
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
