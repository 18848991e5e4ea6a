// api.hip - the exported C ABI (declared in include/mxgemm.h): argument
// validation, device check and kernel choice.  No entry point allocates,
// frees or synchronizes; all work is enqueued on the caller's stream.
#include <string.h>

#include "../../include/mxgemm.h"
#include "mxg_internal.h"

namespace {

// gfx950 check, cached per device (the library runs on one kind of GPU).
constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];  // 0 = unknown, 1 = gfx950, -1 = other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MXG_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return MXG_EUNSUPPORTED;
  int v = __atomic_load_n(&g_arch_ok[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return MXG_EHIP;
    v = (strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    __atomic_store_n(&g_arch_ok[dev], v, __ATOMIC_RELAXED);
  }
  return v == 1 ? MXG_OK : MXG_EUNSUPPORTED;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dim_ok(int64_t d) { return d >= 1 && d <= MXG_MAX_DIM; }

int to_status(hipError_t e) { return e == hipSuccess ? MXG_OK : MXG_EHIP; }

int validate_mx(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const void* C, int64_t M,
                int64_t N, int64_t K, int fmt) {
  if (!A || !SA || !B || !SB || !C) return MXG_EINVAL;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || (K % 32) != 0) return MXG_EINVAL;
  if (fmt < MXG_FMT_FP8_FP8 || fmt > MXG_FMT_FP8_BF6) return MXG_EINVAL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return MXG_EALIGN;
  return MXG_OK;
}

int validate_epi(const float* bias, int act, int out_type) {
  if (act != MXG_ACT_NONE && act != MXG_ACT_GELU) return MXG_EINVAL;
  if (out_type != MXG_OUT_F32 && out_type != MXG_OUT_BF16 && out_type != MXG_OUT_F16) return MXG_EINVAL;
  if (bias != nullptr && !aligned16(bias)) return MXG_EALIGN;
  return MXG_OK;
}

// integer weights (remapped in registers to MFMA operand codes) and FP6
// weights (MFMA operands as stored): the split-K kernel takes them for every
// M the decode and tiled kernels do not
bool remapped_weights(int fmt) {
  return fmt == MXG_FMT_FP8_INT4 || fmt == MXG_FMT_FP8_INT2 || fmt == MXG_FMT_FP8_FP6 || fmt == MXG_FMT_FP8_BF6;
}

// Kernel choice for an MX product (arguments validated): the weight-streaming
// decode kernel (E4M3 activations against E4M3, E2M1, E2M3, E3M2, INT4 or
// INT2 weights), the split-K skinny kernel (the same), or the tiled /
// ping-pong kernels (every 8- and 4-bit float format pair; integer weights,
// and FP6 weights when K is a multiple of 128, on the tiled kernel).  FP6
// weights with other K and more than 64 rows of activations run the split-K
// kernel once per 64 rows (B is read once per 64 rows: a correct path for
// such shapes, not a tuned one).
int run_mx(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const mxg::Epi& e, int64_t M,
           int64_t N, int64_t K, int fmt, hipStream_t st) {
  if (mxg::decode_ok(M, K, fmt, SA, SB, e)) return to_status(mxg::launch_mx_decode(A, SA, B, SB, e, M, N, K, fmt, st));
  // FP6 weights with more rows, K in whole 128-k slices: the tiled kernel
  // (the byte offsets of 128 weight rows stay below 2^31)
  if ((fmt == MXG_FMT_FP8_FP6 || fmt == MXG_FMT_FP8_BF6) && M > mxg::kSkinnyMaxM && K % 128 == 0 && K < (1 << 24))
    return to_status(mxg::launch_mx_tiled(A, SA, B, SB, e, M, N, K, fmt, st));
  // integer weights with more rows: the tiled kernel (any K; in a partial
  // last slice the codes past K are finite and meet zeroed activations)
  if ((fmt == MXG_FMT_FP8_INT4 || fmt == MXG_FMT_FP8_INT2) && M > mxg::kSkinnyMaxM)
    return to_status(mxg::launch_mx_tiled(A, SA, B, SB, e, M, N, K, fmt, st));
  if (remapped_weights(fmt) && M > mxg::kSkinnyMaxM) {
    const int64_t eb = mxg::epi_elem_bytes(e.out);
    for (int64_t m0 = 0; m0 < M; m0 += mxg::kSkinnyMaxM) {
      mxg::Epi ec = e;
      ec.C = (uint8_t*)e.C + m0 * N * eb;
      const int64_t mc = M - m0 < mxg::kSkinnyMaxM ? M - m0 : mxg::kSkinnyMaxM;
      const hipError_t err = mxg::launch_mx_skinny((const uint8_t*)A + m0 * K, SA + m0 * (K / 32), B, SB, ec, mc,
                                                   N, K, fmt, st);
      if (err != hipSuccess) return to_status(err);
    }
    return MXG_OK;
  }
  if (M <= mxg::kSkinnyMaxM &&
      (fmt == MXG_FMT_FP8_FP8 || fmt == MXG_FMT_FP8_FP4 || remapped_weights(fmt))) {
    // K not a multiple of 1024, up to 16 rows, fp32 C: the decode kernel
    // takes the largest multiple of 1024 below K, the split-K kernel adds the
    // rest (with more rows the split-K kernel alone measured faster at
    // N = 4096)
    const int64_t k1 = K - K % 1024;
    const mxg::Epi plain{e.C, nullptr, mxg::kOutF32, mxg::kActNone};
    if (M <= 16 && e.out == mxg::kOutF32 && mxg::decode_ok(M, k1, fmt, SA, SB, plain)) {
      const hipError_t err = mxg::launch_mx_decode(A, SA, B, SB, plain, M, N, K, fmt, st, k1);
      if (err != hipSuccess) return to_status(err);
      return to_status(mxg::launch_mx_skinny(A, SA, B, SB, e, M, N, K, fmt, st, k1));
    }
    return to_status(mxg::launch_mx_skinny(A, SA, B, SB, e, M, N, K, fmt, st));
  }
  return to_status(mxg::launch_mx_tiled(A, SA, B, SB, e, M, N, K, fmt, st));
}

static_assert(MXG_OUT_F32 == mxg::kOutF32 && MXG_OUT_BF16 == mxg::kOutBF16 && MXG_OUT_F16 == mxg::kOutF16,
              "output type ids");
static_assert(MXG_ACT_NONE == mxg::kActNone && MXG_ACT_GELU == mxg::kActGelu, "activation ids");
static_assert(MXG_ELEM_E4M3 == mxg::kFmtFp8 && MXG_ELEM_E5M2 == mxg::kFmtBf8 && MXG_ELEM_E2M1 == mxg::kFmtFp4,
              "element ids are the MFMA format ids");
static_assert(MXG_ELEM_INT4 == mxg::kElemInt4 && MXG_ELEM_INT2 == mxg::kElemInt2, "integer element ids");
static_assert(MXG_ELEM_E2M3 == mxg::kFmtFp6 && MXG_ELEM_E3M2 == mxg::kFmtBf6, "FP6 element ids");
static_assert(MXG_FMT_FP8_FP6 == 8 && MXG_FMT_FP8_BF6 == 9, "FP6 pair ids the split-K launch switches on");

}  // namespace

extern "C" {

const char* mxgemm_status_string(int status) {
  switch (status) {
    case MXG_OK:
      return "ok";
    case MXG_EINVAL:
      return "invalid argument (null pointer, dimension out of range, K not a multiple of 32, or unknown format)";
    case MXG_EALIGN:
      return "data pointer not 16-byte aligned";
    case MXG_EUNSUPPORTED:
      return "device is not gfx950 (MI355X)";
    case MXG_EHIP:
      return "HIP runtime error at launch";
    default:
      return "unknown status";
  }
}

int mxgemm_device_supported(void) {
  const int s = check_device();
  if (s == MXG_OK) return 1;
  if (s == MXG_EUNSUPPORTED) return 0;
  return -s;
}

int mxgemm_quantize(const float* X, int64_t rows, int64_t K, int elem, void* Q, uint8_t* S, void* stream) {
  if (!X || !Q || !S) return MXG_EINVAL;
  if (!dim_ok(rows) || !dim_ok(K) || (K % 32) != 0) return MXG_EINVAL;
  if (elem != MXG_ELEM_E4M3 && elem != MXG_ELEM_E5M2 && elem != MXG_ELEM_E2M1 && elem != MXG_ELEM_INT4 &&
      elem != MXG_ELEM_INT2 && elem != MXG_ELEM_E2M3 && elem != MXG_ELEM_E3M2)
    return MXG_EINVAL;
  if (!aligned16(X) || !aligned16(Q)) return MXG_EALIGN;
  const int d = check_device();
  if (d != MXG_OK) return d;
  return to_status(mxg::launch_quantize(X, rows, K, elem, Q, S, (hipStream_t)stream));
}

int mxgemm_run(const void* A, const uint8_t* scaleA, const void* B, const uint8_t* scaleB, float* C, int64_t M,
               int64_t N, int64_t K, int fmt, void* stream) {
  int s = validate_mx(A, scaleA, B, scaleB, C, M, N, K, fmt);
  if (s != MXG_OK) return s;
  s = check_device();
  if (s != MXG_OK) return s;
  return run_mx(A, scaleA, B, scaleB, mxg::Epi{C, nullptr, mxg::kOutF32, mxg::kActNone}, M, N, K, fmt,
                (hipStream_t)stream);
}

int mxgemm_run_fused(const void* A, const uint8_t* scaleA, const void* B, const uint8_t* scaleB, void* C,
                     int64_t M, int64_t N, int64_t K, int fmt, const float* bias, int act, int out_type,
                     void* stream) {
  int s = validate_mx(A, scaleA, B, scaleB, C, M, N, K, fmt);
  if (s != MXG_OK) return s;
  s = validate_epi(bias, act, out_type);
  if (s != MXG_OK) return s;
  s = check_device();
  if (s != MXG_OK) return s;
  return run_mx(A, scaleA, B, scaleB, mxg::Epi{C, bias, out_type, act}, M, N, K, fmt, (hipStream_t)stream);
}

int mxgemm_epilogue(const float* X, int64_t M, int64_t N, const float* bias, int act, int out_type, void* Y,
                    void* stream) {
  if (!X || !Y) return MXG_EINVAL;
  if (!dim_ok(M) || !dim_ok(N)) return MXG_EINVAL;
  if (!aligned16(X) || !aligned16(Y)) return MXG_EALIGN;
  int s = validate_epi(bias, act, out_type);
  if (s != MXG_OK) return s;
  s = check_device();
  if (s != MXG_OK) return s;
  return to_status(mxg::launch_epilogue(X, M, N, mxg::Epi{Y, bias, out_type, act}, (hipStream_t)stream));
}

int fp16gemm_run(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N, int64_t K, int b_is_nk,
                 void* stream) {
  if (!A || !B || !C) return MXG_EINVAL;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K) || (K % 8) != 0) return MXG_EINVAL;
  if (b_is_nk != 0 && b_is_nk != 1) return MXG_EINVAL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return MXG_EALIGN;
  const int s = check_device();
  if (s != MXG_OK) return s;
  return to_status(mxg::launch_f16_tiled(A, B, C, M, N, K, b_is_nk, (hipStream_t)stream));
}

int mxgemm_run_dequant_fp16(const void* A, const uint8_t* scaleA, const void* B, const uint8_t* scaleB, float* C,
                            int64_t M, int64_t N, int64_t K, int fmt, void* stream) {
  int s = validate_mx(A, scaleA, B, scaleB, C, M, N, K, fmt);
  if (s != MXG_OK) return s;
  if (fmt != MXG_FMT_FP8_FP8) return MXG_EINVAL;
  s = check_device();
  if (s != MXG_OK) return s;
  return to_status(mxg::launch_deq_tiled(A, scaleA, B, scaleB, C, M, N, K, (hipStream_t)stream));
}

}  // extern "C"
