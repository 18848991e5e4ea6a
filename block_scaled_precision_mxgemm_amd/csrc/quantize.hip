// quantize.hip - fp32 rows -> E4M3 or E2M1 codes with one UE8M0 scale per 32
// consecutive K elements.
//
// Rule (one block of 32): amax = max |x|; e = floor(log2 amax) - emax with
// emax = 8 (E4M3, largest finite 448 = 1.75 * 2^8) or 2 (E2M1, 6 = 1.5 * 2^2),
// clamped to [-127, 127], e = -127 for an all-zero block; scale byte e + 127;
// every element x * 2^-e is rounded to nearest, ties to even, and saturated to
// the largest finite magnitude (E4M3 has no infinity and clamps at +-448:
// "Resumo Técnico: RIGEL", section 3, saturation).  A block holding a NaN or
// an infinity gets scale byte 255 (NaN) and zero codes.  One E8M0 scale per 32
// elements along the reduction axis: WWDC26 session 330 summary, section
// "Scale Factor 付き量子化 tensor を作成する".
//
// All arithmetic is integer work on the fp32 bit patterns, so the result does
// not depend on the denormal or rounding mode of the float units.
//
// Work mapping: 8 lanes per block, 4 elements (one 16-byte load) per lane; a
// wave covers 8 consecutive blocks = 1 KiB of input with fully coalesced loads
// and 256 B (E4M3) / 128 B (E2M1) of contiguous code stores; each lane keeps
// four such loads in flight.  The kernel is
// bound by HBM bandwidth: 4 bytes read and 1 + 1/32 (E4M3) or 1/2 + 1/32
// (E2M1) bytes written per element.
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

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

// round(s / 2^sh) with ties to even; s < 2^24.
__device__ __forceinline__ uint32_t rne_shift(uint32_t s, int sh) {
  if (sh <= 0) return s << (-sh);
  if (sh >= 26) return 0u;
  const uint32_t q = s >> sh;
  const uint32_t rem = s & ((1u << sh) - 1u);
  const uint32_t half = 1u << (sh - 1);
  return q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
}

// E4M3 code of x * 2^-e (sign from x).
__device__ __forceinline__ uint32_t encode_e4m3(uint32_t bits, int e) {
  const uint32_t sign = (bits >> 31) << 7;
  const Mag m = split_abs(bits);
  if (m.s == 0) return sign;
  const int base = m.ex - 23 - e;              // |v| = s * 2^base
  const int fl = floor_log2_u(m.s) + base;     // floor(log2 |v|)
  const int qe = max(fl, -6) - 3;              // grid spacing 2^qe
  uint32_t q = rne_shift(m.s, qe - base);      // |v| / 2^qe, rounded
  uint32_t code;
  if (qe == -9) {
    code = q;                                  // subnormal step 2^-9; q = 8 is 2^-6
  } else {
    int ef = qe + 10;                          // biased exponent field (bias 7)
    if (q == 16u) {
      ++ef;
      q = 8u;
    }
    const uint32_t mant = q - 8u;
    if (ef > 15 || (ef == 15 && mant == 7u))
      code = 0x7eu;                            // saturate at 448
    else
      code = ((uint32_t)ef << 3) | mant;
  }
  return code | sign;
}

// E2M1 nibble of x * 2^-e (sign from x).
__device__ __forceinline__ uint32_t encode_e2m1(uint32_t bits, int e) {
  const uint32_t sign = (bits >> 31) << 3;
  const Mag m = split_abs(bits);
  if (m.s == 0) return sign;
  const int base = m.ex - 23 - e;
  const int fl = floor_log2_u(m.s) + base;
  const int qe = max(fl, 0) - 1;
  uint32_t q = rne_shift(m.s, qe - base);
  uint32_t code;
  if (qe == -1) {
    code = q;                                  // 0, 0.5 or (q = 2) 1.0
  } else {
    int ef = qe + 2;                           // biased exponent field (bias 1)
    if (q == 4u) {
      ++ef;
      q = 2u;
    }
    code = (ef > 3) ? 7u : (((uint32_t)ef << 1) | (q - 2u));  // saturate at 6
  }
  return code | sign;
}

// One block of 32: lanes sub = 0..7 of the block hold its elements 4*sub ..
// 4*sub+3 in x; writes the block's codes and (lane 0) its scale byte.
template <int ELEM>
__device__ __forceinline__ void quantize_block(const v4i& x, int64_t blk, int sub, uint8_t* __restrict__ Q,
                                               uint8_t* __restrict__ S) {
  constexpr int kEmax = (ELEM == kFmtFp8) ? 8 : 2;
  uint32_t amax = 0u;
#pragma unroll
  for (int i = 0; i < 4; i++) amax = max(amax, (uint32_t)x[i] & 0x7fffffffu);
  // the 8 lanes of a block are consecutive lanes of one wave
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 4));
  const bool bad = amax >= 0x7f800000u;  // infinity or NaN present
  int e = -127;
  if (amax != 0u) {
    const Mag m = split_abs(amax);
    e = floor_log2_u(m.s) + m.ex - 23 - kEmax;
    e = min(max(e, -127), 127);
  }
  uint32_t c[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    c[i] = bad ? 0u : ((ELEM == kFmtFp8) ? encode_e4m3((uint32_t)x[i], e) : encode_e2m1((uint32_t)x[i], e));
  }
  const int64_t off = blk * 32 + sub * 4;  // element index
  if (ELEM == kFmtFp8) {
    *reinterpret_cast<uint32_t*>(Q + off) = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
  } else {
    *reinterpret_cast<uint16_t*>(Q + (off >> 1)) = (uint16_t)(c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12));
  }
  if (sub == 0) S[blk] = bad ? (uint8_t)255 : (uint8_t)(e + 127);
}

// Rows are contiguous with K % 32 == 0, so block blk (row r, block b) starts
// at element r*K + 32b = 32*blk, and its scale byte is S[blk]: the matrix is
// processed as one flat sequence of blocks.  Each lane keeps kUnroll 16-byte
// loads in flight (grid-stride, all loads issued before any block is
// encoded).
constexpr int kUnroll = 4;

template <int ELEM>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ X, uint8_t* __restrict__ Q,
                                                       uint8_t* __restrict__ S, int64_t total) {
  const int sub = threadIdx.x & 7;
  const int64_t step = ((int64_t)gridDim.x * blockDim.x) >> 3;
  for (int64_t blk0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 3; blk0 < total;
       blk0 += kUnroll * step) {
    v4i x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int64_t blk = blk0 + u * step;
      x[u] = (blk < total) ? *reinterpret_cast<const v4i*>(X + blk * 32 + sub * 4) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; u++) {
      const int64_t blk = blk0 + u * step;
      if (blk < total) quantize_block<ELEM>(x[u], blk, sub, Q, S);
    }
  }
}

}  // namespace

hipError_t launch_quantize(const float* X, int64_t rows, int64_t K, int elem, void* Q, uint8_t* S,
                           hipStream_t stream) {
  const int64_t total = rows * (K >> 5);  // blocks of 32
  int64_t grid = (total * 8 + 255) / 256;
  if (grid > 256 * 32) grid = 256 * 32;
  if (elem == kFmtFp8)
    hipLaunchKernelGGL(quantize_kernel<kFmtFp8>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  else
    hipLaunchKernelGGL(quantize_kernel<kFmtFp4>, dim3((unsigned)grid), dim3(256), 0, stream, X, (uint8_t*)Q, S,
                       total);
  return hipGetLastError();
}

}  // namespace mxg
