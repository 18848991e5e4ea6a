"""CPU oracle for the block-scaled (MX) matrix multiply and its fp16 comparison.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the HIP library and its Python binding) never imports, links or executes
anything here, and this package imports nothing from the product path.

The arithmetic lives in ``mxref.c`` (plain C, float64, OpenMP over output
points only), compiled with gcc into ``oracle/_build/libmxref.so``.  This file
only marshals numpy arrays to it and holds the tolerance gate.

Sources (page title, section):
  * Operand model, one UE8M0 scale per 32 K-elements: "Metal tensors でカスタム
    機械学習オペレーションを最適化する", sections "多平面 tensor" and "Scale
    Factor 付き量子化 tensor を作成する".
  * float64 reference from the exact quantized bytes, per-dtype tolerance gate:
    "Resumo Técnico: RIGEL", section "Metodologia: O Harness RIGEL".
  * E4M3 saturates at +-448 with no infinity; accumulator at least fp32:
    "Resumo Técnico: RIGEL", section 3 "Semântica Numérica e Restrições Ocultas".
  * Plain triple loop: "Treinar LLM em Swift", section "Passo 1".

Every function here is pinned by ``tests/test_oracle_*.py`` against torch's
independent fp8/e8m0 dtypes, the OCP MX E2M1 value list, exact rational brute
force, closed forms and the accumulator-width example the RIGEL summary prints.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

E4M3 = 0
E5M2 = 1
E2M3 = 2
E3M2 = 3
E2M1 = 4
INT4 = 8
INT2 = 9

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxref.c")
_LIB = os.path.join(_HERE, "_build", "libmxref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile mxref.c with gcc (-O2, OpenMP, no FP contraction)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
           "-D_GNU_SOURCE", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.mxref_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.mxref_e4m3_value.restype = ctypes.c_double
    lib.mxref_e5m2_value.argtypes = [ctypes.c_uint8]
    lib.mxref_e5m2_value.restype = ctypes.c_double
    lib.mxref_e2m1_value.argtypes = [ctypes.c_uint8]
    lib.mxref_e2m1_value.restype = ctypes.c_double
    lib.mxref_e2m3_value.argtypes = [ctypes.c_uint8]
    lib.mxref_e2m3_value.restype = ctypes.c_double
    lib.mxref_e3m2_value.argtypes = [ctypes.c_uint8]
    lib.mxref_e3m2_value.restype = ctypes.c_double
    lib.mxref_int4_value.argtypes = [ctypes.c_uint8]
    lib.mxref_int4_value.restype = ctypes.c_double
    lib.mxref_int2_value.argtypes = [ctypes.c_uint8]
    lib.mxref_int2_value.restype = ctypes.c_double
    lib.mxref_ue8m0_value.argtypes = [ctypes.c_uint8]
    lib.mxref_ue8m0_value.restype = ctypes.c_double
    lib.mxref_fp16_value.argtypes = [ctypes.c_uint16]
    lib.mxref_fp16_value.restype = ctypes.c_double
    lib.mxref_quantize.argtypes = [p, i64, i64, ci, p, p]
    lib.mxref_quantize.restype = ci
    lib.mxref_gemm.argtypes = [p, p, ci, p, p, ci, i64, i64, i64, p, p, p]
    lib.mxref_gemm.restype = ci
    lib.mxref_gemm_points.argtypes = [p, p, ci, p, p, ci, i64, i64, i64, p, p, i64, p, p, p]
    lib.mxref_gemm_points.restype = ci
    lib.mxref_fp16_gemm.argtypes = [p, p, i64, i64, i64, ci, p, p]
    lib.mxref_fp16_gemm.restype = ci
    lib.mxref_fp16_gemm_points.argtypes = [p, p, i64, i64, i64, ci, p, p, i64, p, p]
    lib.mxref_fp16_gemm_points.restype = ci
    lib.mxref_gelu.argtypes = [ctypes.c_double]
    lib.mxref_gelu.restype = ctypes.c_double
    lib.mxref_round_bf16.argtypes = [ctypes.c_double]
    lib.mxref_round_bf16.restype = ctypes.c_double
    lib.mxref_round_f16.argtypes = [ctypes.c_double]
    lib.mxref_round_f16.restype = ctypes.c_double
    lib.mxref_epilogue.argtypes = [p, p, i64, p, ci, p]
    lib.mxref_epilogue.restype = ci
    lib.mxref_num_threads.argtypes = []
    lib.mxref_num_threads.restype = ci
    lib.mxref_set_num_threads.argtypes = [ci]
    lib.mxref_set_num_threads.restype = ci
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS or all cores)."""
    return int(_load().mxref_num_threads())


def set_num_threads(n: int) -> int:
    """Set the threads of the oracle's OpenMP loops; returns the count in effect."""
    return int(_load().mxref_set_num_threads(int(n)))


# ----------------------------------------------------------------- tables

def e4m3_table() -> np.ndarray:
    """float64[256]: value of every E4M3 code (NaN for 0x7F and 0xFF)."""
    lib = _load()
    return np.array([lib.mxref_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e5m2_table() -> np.ndarray:
    """float64[256]: value of every E5M2 code (+-inf for 0x7C / 0xFC, NaN for
    exponent field 31 with a nonzero mantissa)."""
    lib = _load()
    return np.array([lib.mxref_e5m2_value(c) for c in range(256)], dtype=np.float64)


def e2m1_table() -> np.ndarray:
    """float64[16]: value of every E2M1 nibble."""
    lib = _load()
    return np.array([lib.mxref_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m3_table() -> np.ndarray:
    """float64[64]: value of every E2M3 (FP6) code."""
    lib = _load()
    return np.array([lib.mxref_e2m3_value(c) for c in range(64)], dtype=np.float64)


def e3m2_table() -> np.ndarray:
    """float64[64]: value of every E3M2 (FP6) code."""
    lib = _load()
    return np.array([lib.mxref_e3m2_value(c) for c in range(64)], dtype=np.float64)


def int4_table() -> np.ndarray:
    """float64[16]: value of every two's complement INT4 code (-8..7)."""
    lib = _load()
    return np.array([lib.mxref_int4_value(c) for c in range(16)], dtype=np.float64)


def int2_table() -> np.ndarray:
    """float64[4]: value of every two's complement INT2 code (-2..1)."""
    lib = _load()
    return np.array([lib.mxref_int2_value(c) for c in range(4)], dtype=np.float64)


def ue8m0_table() -> np.ndarray:
    """float64[256]: 2^(e-127) for every scale byte, NaN for 255."""
    lib = _load()
    return np.array([lib.mxref_ue8m0_value(c) for c in range(256)], dtype=np.float64)


def fp16_value(bits: int) -> float:
    return float(_load().mxref_fp16_value(bits))


def row_bytes(K: int, elem: int) -> int:
    """Bytes per operand row: K for E4M3 and E5M2, K/2 for packed E2M1 and
    INT4, K/4 for packed INT2, 3K/4 for packed E2M3 and E3M2."""
    if elem in (E2M1, INT4):
        return K // 2
    if elem == INT2:
        return K // 4
    if elem in (E2M3, E3M2):
        return K // 4 * 3
    return K


# --------------------------------------------------------------- quantize

def quantize(x: np.ndarray, elem: int):
    """Quantize fp32 rows (K contiguous) to (codes uint8, scales uint8).

    codes: rows x K (E4M3, E5M2), rows x K/2 (E2M1, INT4: even k in the low
    nibble), rows x K/4 (INT2: k in bits 2 (k mod 4)) or rows x 3K/4 (E2M3,
    E3M2: k in bits 6k .. 6k+5 of the row, little-endian); scales: rows x K/32
    UE8M0 bytes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, K = x.shape
    q = np.zeros((rows, row_bytes(K, elem)), dtype=np.uint8)
    s = np.zeros((rows, K // 32), dtype=np.uint8)
    rc = _load().mxref_quantize(_ptr(x), rows, K, elem, _ptr(q), _ptr(s))
    if rc != 0:
        raise ValueError("oracle quantize: bad arguments (K %% 32 must be 0, elem E4M3/E5M2/E2M3/E3M2/E2M1/INT4/INT2)")
    return q, s


# ------------------------------------------------------------------- GEMM

def _check_operand(q, s, rows, K, elem, name):
    if q.dtype != np.uint8 or s.dtype != np.uint8:
        raise TypeError(name + ": codes and scales must be uint8")
    if q.shape != (rows, row_bytes(K, elem)) or s.shape != (rows, K // 32):
        raise ValueError(name + ": shape mismatch")


def mx_gemm(a_q, a_s, elem_a, b_q, b_s, elem_b, M, N, K, points=None, step_max=False):
    """float64 reference C and the magnitude sum |A||B| (same shape).

    A is M x K codes with M x K/32 scales; B is N x K codes with N x K/32
    scales (both K contiguous).  With ``points=(I, J)`` only those output
    elements are computed and 1-D arrays are returned.  With
    ``step_max=True`` a third array is returned: for each output element the
    sum, over the 128-element steps of K (k = 128t .. 128t+127), of the
    largest scaled product magnitude in the step (a tolerance input, see
    ``gate``).
    """
    a_q = np.ascontiguousarray(a_q)
    a_s = np.ascontiguousarray(a_s)
    b_q = np.ascontiguousarray(b_q)
    b_s = np.ascontiguousarray(b_s)
    _check_operand(a_q, a_s, M, K, elem_a, "A")
    _check_operand(b_q, b_s, N, K, elem_b, "B")
    lib = _load()
    if points is None:
        C = np.empty((M, N), dtype=np.float64)
        ABS = np.empty((M, N), dtype=np.float64)
        SMAX = np.empty((M, N), dtype=np.float64) if step_max else None
        rc = lib.mxref_gemm(_ptr(a_q), _ptr(a_s), elem_a, _ptr(b_q), _ptr(b_s), elem_b,
                            M, N, K, _ptr(C), _ptr(ABS), None if SMAX is None else _ptr(SMAX))
    else:
        I = np.ascontiguousarray(points[0], dtype=np.int64)
        J = np.ascontiguousarray(points[1], dtype=np.int64)
        C = np.empty(I.shape[0], dtype=np.float64)
        ABS = np.empty(I.shape[0], dtype=np.float64)
        SMAX = np.empty(I.shape[0], dtype=np.float64) if step_max else None
        rc = lib.mxref_gemm_points(_ptr(a_q), _ptr(a_s), elem_a, _ptr(b_q), _ptr(b_s), elem_b,
                                   M, N, K, _ptr(I), _ptr(J), I.shape[0], _ptr(C), _ptr(ABS),
                                   None if SMAX is None else _ptr(SMAX))
    if rc != 0:
        raise ValueError("oracle mx_gemm: bad arguments")
    return (C, ABS, SMAX) if step_max else (C, ABS)


def fp16_gemm(a_bits, b_bits, M, N, K, b_is_nk, points=None):
    """float64 reference for C = A B on binary16 inputs (given as uint16 bits).

    A is M x K row-major; B is K x N row-major (b_is_nk=0) or N x K (b_is_nk=1).
    """
    a = np.ascontiguousarray(a_bits).view(np.uint16)
    b = np.ascontiguousarray(b_bits).view(np.uint16)
    if a.shape != (M, K) or b.shape != ((N, K) if b_is_nk else (K, N)):
        raise ValueError("oracle fp16_gemm: shape mismatch")
    lib = _load()
    if points is None:
        C = np.empty((M, N), dtype=np.float64)
        ABS = np.empty((M, N), dtype=np.float64)
        rc = lib.mxref_fp16_gemm(_ptr(a), _ptr(b), M, N, K, int(b_is_nk), _ptr(C), _ptr(ABS))
    else:
        I = np.ascontiguousarray(points[0], dtype=np.int64)
        J = np.ascontiguousarray(points[1], dtype=np.int64)
        C = np.empty(I.shape[0], dtype=np.float64)
        ABS = np.empty(I.shape[0], dtype=np.float64)
        rc = lib.mxref_fp16_gemm_points(_ptr(a), _ptr(b), M, N, K, int(b_is_nk),
                                        _ptr(I), _ptr(J), I.shape[0], _ptr(C), _ptr(ABS))
    if rc != 0:
        raise ValueError("oracle fp16_gemm: bad arguments")
    return C, ABS


# ------------------------------------------------------------------- gate

U = 2.0 ** -24  # unit roundoff of fp32


def gate(c_test, c_ref, abs_ref, K, step_max=None, kappa=0.0):
    """Checksum gate: for every element

        |c_test - c_ref| <= K * 2^-24 * sum|a b|  [+ kappa * step_max]

    NaN positions identical, +-Inf positions and signs identical.

    The fp8 x fp8 (or fp4, fp16) products times power-of-two scales are exact
    in fp32, so with fp32 accumulation the only admissible error is
    accumulation error: the classical recursive-summation bound with K terms
    (the default, kappa = 0).  A matrix unit that adds the products of one
    128-element step in a single operation may align them to the step's
    largest product and drop low bits; such a path states its per-step
    error, in units of that step's largest product magnitude, as ``kappa``
    and passes ``step_max`` (from ``mx_gemm(..., step_max=True)``).  One
    tolerance per data path, as RIGEL's gate keeps one per data type
    ("Resumo Técnico: RIGEL", section "Metodologia: O Harness RIGEL").

    Returns a dict with 'ok', 'n_bad', 'max_ratio' (error over the strict
    K-term bound, reported whatever the tolerance), 'max_ratio_tol' (error
    over the tolerance applied), 'nan_mismatch', 'inf_mismatch', 'n_exact'.
    """
    t = np.asarray(c_test, dtype=np.float64)
    r = np.asarray(c_ref, dtype=np.float64)
    a = np.asarray(abs_ref, dtype=np.float64)
    if t.shape != r.shape or r.shape != a.shape:
        raise ValueError("gate: shape mismatch")
    if kappa != 0.0 and (step_max is None or np.shape(step_max) != r.shape):
        raise ValueError("gate: kappa needs step_max of the reference's shape")
    nan_t, nan_r = np.isnan(t), np.isnan(r)
    nan_mismatch = int(np.count_nonzero(nan_t != nan_r))
    inf_t, inf_r = np.isinf(t), np.isinf(r)
    inf_mismatch = int(np.count_nonzero((inf_t != inf_r) | (inf_t & inf_r & (np.sign(t) != np.sign(r)))))
    fin = ~(nan_t | nan_r | inf_t | inf_r)
    strict = K * U * a[fin]
    tol = strict if kappa == 0.0 else strict + kappa * np.asarray(step_max, dtype=np.float64)[fin]
    err = np.abs(t[fin] - r[fin])
    bad = err > tol

    def _ratio(bound):
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(bound > 0, err / np.where(bound > 0, bound, 1.0), np.where(err > 0, np.inf, 0.0))
        return float(q.max()) if q.size else 0.0

    n_exact = int(np.count_nonzero(t[fin] == r[fin].astype(np.float32).astype(np.float64)))
    n_bad = int(np.count_nonzero(bad)) + nan_mismatch + inf_mismatch
    return {
        "ok": n_bad == 0,
        "n_bad": n_bad,
        "n": int(t.size),
        "max_ratio": _ratio(strict),
        "max_ratio_tol": _ratio(tol),
        "nan_mismatch": nan_mismatch,
        "inf_mismatch": inf_mismatch,
        "n_exact": n_exact,
    }


# --------------------------------------------------------------- epilogue
# The output step of the fused GEMM: y = act(c + bias[col]) in float64, then
# the output type.  "Resumo Técnico: RIGEL", section "4. Oportunidades de
# Otimização" (GEMM fused with bias and GELU).  Reading: GELU(y) = y Phi(y).

OUT_F32, OUT_BF16, OUT_F16 = 0, 1, 2
ACT_NONE, ACT_GELU = 0, 1

# Largest slope of GELU: d/dy [y Phi(y)] = Phi(y) + y phi(y), maximal at
# y = sqrt(2): Phi(sqrt 2) + sqrt(2) phi(sqrt 2) = 1.12897...
GELU_LIPSCHITZ = 1.129
# Error of the GPU's GELU in units of |y| / 2 (absolute error of its erf):
# Abramowitz & Stegun 7.1.26 (1.5e-7) plus its fp32 evaluation (reciprocal,
# five fma / mul, exp, the final 2 - E: at most 8 roundings of values <= 2).
GELU_ERF_ERR = 1.5e-7 + 8 * 2.0 ** -23


def gelu(y):
    lib = _load()
    return np.array([lib.mxref_gelu(float(v)) for v in np.ravel(y)], dtype=np.float64).reshape(np.shape(y))


def round_out(v, out_type):
    """float64 values rounded (RNE, overflow to inf) to the output type."""
    if out_type == OUT_F32:
        with np.errstate(over="ignore", invalid="ignore"):
            return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
    lib = _load()
    f = lib.mxref_round_bf16 if out_type == OUT_BF16 else lib.mxref_round_f16
    return np.array([f(float(x)) for x in np.ravel(v)], dtype=np.float64).reshape(np.shape(v))


def epilogue(c, cols, bias, act):
    """act(c + bias[cols]) in float64 (bias None: no bias)."""
    c = np.ascontiguousarray(c, dtype=np.float64).ravel()
    cols = np.ascontiguousarray(cols, dtype=np.int64).ravel()
    y = np.empty_like(c)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    rc = _load().mxref_epilogue(_ptr(c), _ptr(cols), c.shape[0], None if b is None else _ptr(b), int(act), _ptr(y))
    if rc != 0:
        raise ValueError("oracle epilogue: bad arguments")
    return y


def _half_ulp(a, out_type):
    """Half the spacing of the output format at magnitude a (a >= 0)."""
    P, EMIN = {OUT_F32: (24, -126), OUT_BF16: (8, -126), OUT_F16: (11, -14)}[out_type]
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, EMIN)
    # one binade up as well, so a value that rounds up across a power of two
    # is covered
    return np.ldexp(1.0, (e + 1 - P).astype(np.int64)) * 0.5 * 2.0


def epilogue_gate(out_vals, c_ref, abs_ref, K, cols, bias, act, out_type, step_max=None, kappa=0.0):
    """Gate for the fused output: |out - act(c_ref + bias)| within

      d_c   = K 2^-24 sum|a b| [+ kappa step_max]  (the GEMM's bound, as in gate())
      d_y   = d_c + 2^-24 |y|                     (the fp32 bias add)
      d_g   = L d_y + |y|/2 (GELU_ERF_ERR + 2^-22) + 2^-23 |g|   (with GELU;
              L the largest slope of GELU)
      + half an ulp of the output type at the value (its final rounding),
    with |y| and |g| taken as the larger of the reference and the output.
    NaN positions must match; infinities must match in position and sign,
    where the reference's infinities are those of the exact value rounded to
    the output type (beyond its range it is +-inf).
    """
    t = np.asarray(out_vals, dtype=np.float64).ravel()
    c = np.asarray(c_ref, dtype=np.float64).ravel()
    ab = np.asarray(abs_ref, dtype=np.float64).ravel()
    ref = epilogue(c, cols, bias, act)
    y_ref = c if bias is None else c + np.asarray(bias, dtype=np.float64)[np.asarray(cols).ravel()]
    ref_r = round_out(ref, out_type)
    nan_t, nan_r = np.isnan(t), np.isnan(ref)
    nan_mismatch = int(np.count_nonzero(nan_t != nan_r))
    inf_t, inf_r = np.isinf(t), np.isinf(ref_r)
    inf_mismatch = int(np.count_nonzero((inf_t != inf_r) | (inf_t & inf_r & (np.sign(t) != np.sign(ref_r)))))
    fin = ~(nan_t | nan_r | inf_t | inf_r)
    t, ref, c, ab, y_ref = t[fin], ref[fin], c[fin], ab[fin], y_ref[fin]
    d = K * U * ab
    if kappa != 0.0:
        d = d + kappa * np.asarray(step_max, dtype=np.float64).ravel()[fin]
    ymag = np.maximum(np.abs(y_ref), np.abs(t))
    if bias is not None:
        d = d + U * ymag
    if act == ACT_GELU:
        gmag = np.maximum(np.abs(ref), np.abs(t))
        d = GELU_LIPSCHITZ * d + 0.5 * ymag * (GELU_ERF_ERR + 2.0 ** -22) + 2.0 ** -23 * gmag
    tol = d + _half_ulp(np.maximum(np.abs(ref), np.abs(t)), out_type)
    err = np.abs(t - ref)
    bad = err > tol
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err > 0, np.inf, 0.0))
    n_bad = int(np.count_nonzero(bad)) + nan_mismatch + inf_mismatch
    return {"ok": n_bad == 0, "n_bad": n_bad, "n": int(np.size(out_vals)),
            "max_ratio": float(ratio.max()) if ratio.size else 0.0,
            "nan_mismatch": nan_mismatch, "inf_mismatch": inf_mismatch}
