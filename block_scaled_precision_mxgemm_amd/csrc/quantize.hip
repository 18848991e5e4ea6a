// quantize.hip - fp32 rows -> E4M3, E5M2, E2M1, E2M3, E3M2, INT4 or INT2
// codes with one UE8M0 scale per 32 consecutive K elements.
//
// Rule (one block of 32): amax = max |x|; e = floor(log2 amax) - emax with
// emax = 8 (E4M3, largest finite 448 = 1.75 * 2^8), 15 (E5M2, 57344 =
// 1.75 * 2^15) or 2 (E2M1, 6 = 1.5 * 2^2),
// clamped to [-127, 127], e = -127 for an all-zero block; scale byte e + 127;
// every element x * 2^-e is rounded to nearest, ties to even, and saturated to
// the largest finite magnitude (E4M3 has no infinity and clamps at +-448:
// "Resumo Técnico: RIGEL", section 3, saturation; E5M2 is saturated the same
// way inside a block, although a plain E5M2 cast overflows to infinity).  A block holding a NaN or
// an infinity gets scale byte 255 (NaN) and zero codes.  One E8M0 scale per 32
// elements along the reduction axis: WWDC26 session 330 summary, section
// "Scale Factor 付き量子化 tensor を作成する".  The integer formats (two's
// complement INT4 -8..7, INT2 -2..1: the 4-bit and 2-bit integer tensor
// types of the same summary, section "量子化データ型のネイティブサポート")
// take emax = 2 and 0 (the largest power of two of the range) and are
// rounded to the nearest integer, ties to even, saturated to the range.
// The FP6 formats (the 6-bit float operands of the scaled matrix unit; the
// pages give no layout, so the OCP Microscaling definitions are taken) take
// emax = 2 (E2M3, 7.5 = 1.875 * 2^2) and 4 (E3M2, 28 = 1.75 * 2^4), and are
// packed little-endian, element k at bits 6k .. 6k+5 of its row.
//
// The block exponent is integer work on the fp32 bit patterns.  E4M3, E5M2
// and E2M1 codes come from gfx950's conversion instructions (fp32 -> OCP
// E4M3 / E5M2 pairs, fp32 -> E2M1 pairs) applied to x * 2^-e: the scaling is
// exact (a power of two; a product small enough to lose bits as an fp32
// subnormal lies far below half the format's smallest subnormal, so its code
// is a signed zero either way), the value is first clamped to the largest
// finite magnitude, which gives the saturation, and the conversion rounds to
// nearest even in the default float mode of a kernel (round to nearest,
// fp32 subnormals kept).  The integer and FP6 codes are computed in integer
// arithmetic (encode_mag below).  Both routes are bit-exact against the
// float64 reference on every E4M3 tie, every mantissa at the exponents where
// the rounding regime changes, and blocks of subnormals.  The integer route
// for E4M3 ran the 8192 x 8192 quantization at 66 us; the conversions bring it
// to the memory stream (the encode, ~25 VALU instructions per element, had
// been the limit).
//
// Work mapping: 8 lanes per block, 4 elements (one 16-byte load) per lane; a
// wave covers 8 consecutive blocks = 1 KiB of input with fully coalesced loads
// and 256 B (E4M3) / 128 B (E2M1) of contiguous code stores; each lane keeps
// four such loads in flight (see quantize_kernel for the workgroup's range).
// The kernel is bound by HBM bandwidth: 4 bytes read and 1 + 1/32 (E4M3) or
// 1/2 + 1/32 (E2M1) bytes written per element.
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

// DPP lane patterns (gfx9 encodings): quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], and row_half_mirror (lane i of each 8 takes lane 7 - i).
constexpr int kDppSwap1 = 0xB1;
constexpr int kDppSwap2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;

// |x| = s * 2^(ex - 23) with s < 2^24; s = 0 for zero.
struct Mag {
  uint32_t s;
  int ex;
};

__device__ __forceinline__ Mag split_abs(uint32_t bits) {
  const uint32_t bexp = (bits >> 23) & 0xffu;
  const uint32_t mant = bits & 0x7fffffu;
  Mag m;
  if (bexp == 0) {
    m.s = mant;
    m.ex = -126;
  } else {
    m.s = mant | 0x800000u;
    m.ex = (int)bexp - 127;
  }
  return m;
}

__device__ __forceinline__ int floor_log2_u(uint32_t s) { return 31 - __clz((int)s); }

// Code of x * 2^-e in a format with MBITS mantissa bits whose smallest normal
// exponent is KMIN, saturated at MAXCODE (sign not included), branch-free:
//   |x| = m * 2^(k - 23) with m in [2^23, 2^24) (subnormal x normalized first)
//   so k = floor(log2 |x * 2^-e|);
//   normal results (k >= KMIN): q = m / 2^(23 - MBITS) rounded to nearest, ties
//   to even, lies in [2^MBITS, 2^(MBITS+1)], and the code is
//   ((k - KMIN) << MBITS) + q, the carry of q = 2^(MBITS+1) running into the
//   exponent field by itself;
//   subnormal results (k < KMIN): the spacing is fixed at 2^(KMIN - MBITS), so
//   q = m / 2^(23 - MBITS + KMIN - k) rounded the same way is the code, and
//   q = 2^MBITS is the smallest normal;
//   zero (m = 0) gives q = 0, shifts past 31 bits give 0, and every code
//   above MAXCODE (the largest finite value) saturates to it.
template <int MBITS, int KMIN, uint32_t MAXCODE>
__device__ __forceinline__ uint32_t encode_mag(uint32_t bits, int e) {
  const uint32_t ex = (bits >> 23) & 0xffu;
  const uint32_t mant = bits & 0x7fffffu;
  const uint32_t lz = (uint32_t)__clz((int)mant) - 8u;  // 24 for mant = 0
  const bool sub = ex == 0u;
  const uint32_t m = sub ? (mant << lz) : (mant | 0x800000u);
  const int k = (sub ? 1 - (int)lz : (int)ex) - 127 - e;
  const int t = k - KMIN;
  const uint32_t sh = (uint32_t)min(23 - MBITS + max(-t, 0), 31);
  const uint32_t lsb = (m >> sh) & 1u;
  const uint32_t q = (m + ((1u << (sh - 1u)) - 1u) + lsb) >> sh;
  const uint32_t code = q + ((uint32_t)max(t, 0) << MBITS);
  return min(code, MAXCODE);
}

// FP6: E2M3 (bias 1, 3 mantissa bits, largest 7.5 = 0x1F) and E3M2 (bias 3,
// 2 mantissa bits, largest 28 = 0x1F), sign in bit 5.
__device__ __forceinline__ uint32_t encode_e2m3(uint32_t bits, int e) {
  return encode_mag<3, 0, 0x1Fu>(bits, e) | ((bits >> 31) << 5);
}
__device__ __forceinline__ uint32_t encode_e3m2(uint32_t bits, int e) {
  return encode_mag<2, -2, 0x1Fu>(bits, e) | ((bits >> 31) << 5);
}

// Two's complement integer code of x * 2^-e in BITS bits: a "format" whose
// spacing is 1 everywhere (KMIN = MBITS, so every value takes the subnormal
// branch of encode_mag) rounds |x * 2^-e| to the nearest integer, ties to
// even; positive values saturate at 2^(BITS-1) - 1, negative ones at
// -2^(BITS-1).
template <int BITS>
__device__ __forceinline__ uint32_t encode_int(uint32_t bits, int e) {
  constexpr int MB = BITS - 1;                       // |x * 2^-e| < 2^(BITS-1) up to rounding
  constexpr uint32_t kNeg = 1u << (BITS - 1);        // largest negative magnitude
  const uint32_t q = encode_mag<MB, MB, kNeg>(bits, e);
  const bool neg = (bits >> 31) != 0u;
  const uint32_t mag = neg ? q : min(q, kNeg - 1u);
  return (neg ? 0u - mag : mag) & ((1u << BITS) - 1u);
}

// One block of 32: lanes sub = 0..7 of the block hold its elements 4*sub ..
// 4*sub+3 in x; writes the block's codes and (lane 0) its scale byte.
template <int ELEM>
__device__ __forceinline__ void quantize_block(const v4i& x, int64_t blk, int sub, uint8_t* __restrict__ Q,
                                               uint8_t* __restrict__ S) {
  constexpr int kEmax = (ELEM == kFmtFp8)   ? 8
                        : (ELEM == kFmtBf8) ? 15
                        : (ELEM == kElemInt2) ? 0
                        : (ELEM == kFmtBf6)   ? 4
                                              : 2;  // E2M1, INT4, E2M3
  uint32_t amax = 0u;
#pragma unroll
  for (int i = 0; i < 4; i++) amax = max(amax, (uint32_t)x[i] & 0x7fffffffu);
  // the 8 lanes of a block are consecutive lanes of one wave, half a DPP
  // row: swap neighbours, swap pairs, then mirror the two quads (register
  // moves, where a lane shuffle would go through the LDS crossbar)
  amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, kDppSwap1, 0xF, 0xF, false));
  amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, kDppSwap2, 0xF, 0xF, false));
  amax = max(amax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)amax, kDppHalfMirror, 0xF, 0xF, false));
  const bool bad = amax >= 0x7f800000u;  // infinity or NaN present
  int e = -127;
  if (amax != 0u) {
    const Mag m = split_abs(amax);
    e = floor_log2_u(m.s) + m.ex - 23 - kEmax;
    e = min(max(e, -127), 127);
  }
  const int64_t off = blk * 32 + sub * 4;  // element index
  if constexpr (ELEM == kFmtFp8 || ELEM == kFmtBf8 || ELEM == kFmtFp4) {
    constexpr float kMax = ELEM == kFmtFp8 ? 448.f : ELEM == kFmtBf8 ? 57344.f : 6.f;
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; i++) y[i] = __builtin_amdgcn_fmed3f(ldexpf(__int_as_float(x[i]), -e), -kMax, kMax);
    // the codes are written once and read by a later GEMM: non-temporal
    // stores keep them from displacing the input stream in the caches
    if constexpr (ELEM == kFmtFp4) {
      uint32_t v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y[0], y[1], 1.0f, 0);
      v = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(v, y[2], y[3], 1.0f, 1);
      __builtin_nontemporal_store((uint16_t)(bad ? 0u : v), reinterpret_cast<uint16_t*>(Q + (off >> 1)));
    } else {
      int v;
      if constexpr (ELEM == kFmtFp8) {
        v = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], v, true);
      } else {
        v = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
        v = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], v, true);
      }
      __builtin_nontemporal_store(bad ? 0u : (uint32_t)v, reinterpret_cast<uint32_t*>(Q + off));
    }
    if (sub == 0) S[blk] = bad ? (uint8_t)255 : (uint8_t)(e + 127);
    return;
  }
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    c[i] = bad ? 0u
               : (ELEM == kElemInt4) ? encode_int<4>((uint32_t)x[i], e)
               : (ELEM == kElemInt2) ? encode_int<2>((uint32_t)x[i], e)
               : (ELEM == kFmtFp6)   ? encode_e2m3((uint32_t)x[i], e)
                                     : encode_e3m2((uint32_t)x[i], e);
  }
  // The codes are written once and read by a later GEMM: non-temporal
  // stores keep them from displacing the input stream in the caches (E4M3
  // 8192 x 8192: 80 against 89-93 us, measured)
  if (ELEM == kElemInt2) {
    __builtin_nontemporal_store((uint8_t)(c[0] | (c[1] << 2) | (c[2] << 4) | (c[3] << 6)), Q + (off >> 2));
  } else if (ELEM == kFmtFp6 || ELEM == kFmtBf6) {
    // four 6-bit codes = 3 bytes at byte 3/4 of the element index
    const uint32_t v = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18);
    uint8_t* q = Q + (off >> 2) * 3;
    __builtin_nontemporal_store((uint8_t)v, q);
    __builtin_nontemporal_store((uint8_t)(v >> 8), q + 1);
    __builtin_nontemporal_store((uint8_t)(v >> 16), q + 2);
  } else {
    __builtin_nontemporal_store((uint16_t)(c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12)),
                                reinterpret_cast<uint16_t*>(Q + (off >> 1)));
  }
  if (sub == 0) S[blk] = bad ? (uint8_t)255 : (uint8_t)(e + 127);
}

// Rows are contiguous with K % 32 == 0, so block blk (row r, block b) starts
// at element r*K + 32b = 32*blk, and its scale byte is S[blk]: the matrix is
// processed as one flat sequence of blocks.  A workgroup takes 128
// consecutive blocks (16 KiB of input); its load u (of kUnroll, all issued
// before any block is encoded) covers blocks 32u .. 32u+31 of them, so every
// load instruction of the workgroup reads 4 KiB contiguous.  (Loads spread
// over the matrix, 32 MiB apart per lane, were faster only while the integer
// encoder limited the kernel: E4M3 8192 x 8192 with the input read from HBM,
// 64.5 against 56.8 us.)
constexpr int kUnroll = 4;
constexpr int kBlocksPerGroup = 32 * kUnroll;

template <int ELEM>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ X, uint8_t* __restrict__ Q,
                                                       uint8_t* __restrict__ S, int64_t total) {
  const int sub = threadIdx.x & 7;
  for (int64_t g = blockIdx.x; g * kBlocksPerGroup < total; g += gridDim.x) {
    const int64_t b0 = g * kBlocksPerGroup + (threadIdx.x >> 3);
    v4i x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int64_t blk = b0 + 32 * u;
      x[u] = (blk < total) ? *reinterpret_cast<const v4i*>(X + blk * 32 + sub * 4) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int64_t blk = b0 + 32 * u;
      if (blk < total) quantize_block<ELEM>(x[u], blk, sub, Q, S);
    }
  }
}

}  // namespace

hipError_t launch_quantize(const float* X, int64_t rows, int64_t K, int elem, void* Q, uint8_t* S,
                           hipStream_t stream) {
  const int64_t total = rows * (K >> 5);  // blocks of 32
  // one workgroup per 128 blocks, at most 64 per CU (grid-stride beyond)
  int64_t grid = (total + kBlocksPerGroup - 1) / kBlocksPerGroup;
  if (grid > 256 * 64) grid = 256 * 64;
  if (elem == kFmtFp8)
    hipLaunchKernelGGL(quantize_kernel<kFmtFp8>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  else if (elem == kFmtBf8)
    hipLaunchKernelGGL(quantize_kernel<kFmtBf8>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  else if (elem == kElemInt4)
    hipLaunchKernelGGL(quantize_kernel<kElemInt4>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  else if (elem == kElemInt2)
    hipLaunchKernelGGL(quantize_kernel<kElemInt2>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  else if (elem == kFmtFp6)
    hipLaunchKernelGGL(quantize_kernel<kFmtFp6>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  else if (elem == kFmtBf6)
    hipLaunchKernelGGL(quantize_kernel<kFmtBf6>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  else
    hipLaunchKernelGGL(quantize_kernel<kFmtFp4>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  return hipGetLastError();
}

}  // namespace mxg
