// mxg_epilogue.h - the output step shared by the MX GEMM kernels and the
// stand-alone epilogue kernel: an optional per-column fp32 bias, an optional
// GELU, and the output element type (fp32, bf16 or fp16), applied to the
// fp32 accumulators in registers before the only store of C.  Fusing bias and
// GELU into the GEMM's epilogue so that C makes one trip to memory is the
// optimization "Resumo Técnico: RIGEL", section "4. Oportunidades de
// Otimização", measures against the decomposed path.
//
// Order of operations per element (all in fp32, round to nearest even):
//   y = acc + bias[n]           (skipped without a bias)
//   y = GELU(y)                 (skipped without the activation)
//   C[m][n] = y converted to the output type (RNE; overflow gives +-inf,
//             NaN stays NaN)
#pragma once

#include "mxg_device.h"

namespace mxg {

constexpr int kOutF32 = 0;
constexpr int kOutBF16 = 1;
constexpr int kOutF16 = 2;
constexpr int kActNone = 0;
constexpr int kActGelu = 1;

struct Epi {
  void* C;            // M x N row-major, elements of type `out`
  const float* bias;  // N fp32 values, or nullptr
  int out;            // kOutF32 / kOutBF16 / kOutF16
  int act;            // kActNone / kActGelu
};

__host__ __device__ inline int epi_elem_bytes(int out) { return out == kOutF32 ? 4 : 2; }
__device__ __forceinline__ bool epi_plain(Epi e) {
  return e.out == kOutF32 && e.act == kActNone && e.bias == nullptr;
}

// GELU(y) = y * Phi(y) = y/2 * (1 + erf(y / sqrt(2))).  erf(x) for x >= 0
// from Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x), absolute error <= 1.5e-7.  1 + erf(y/sqrt 2) is formed
// as 2 - E for y >= 0 and as E for y < 0 (E = the t-polynomial times
// exp(-x^2)), so no cancellation occurs for negative y.  GELU(-inf) is NaN
// (0 * inf), as the formula gives in IEEE arithmetic.
__device__ __forceinline__ float gelu(float y) {
  const float x = fabsf(y) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, x, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f), -0.284496736f),
               0.254829592f);
  const float E = poly * __expf(-x * x);
  const float one_plus_erf = (y >= 0.0f) ? 2.0f - E : E;
  return 0.5f * y * one_plus_erf;
}

// fp32 -> bf16 bits, round to nearest even (gfx950's conversion
// instruction); NaN stays a NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// fp32 -> fp16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint32_t f16_bits(float f) {
  const _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// bias (4 columns n .. n+3; `vec`: all four exist and are 16-byte aligned)
// and activation applied to v
__device__ __forceinline__ v4f epi_apply(Epi e, int64_t N, int n, v4f v, bool vec) {
  if (e.bias != nullptr) {
    if (vec) {
      v += *reinterpret_cast<const v4f*>(e.bias + n);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (n + i < N) v[i] += e.bias[n + i];
    }
  }
  if (e.act == kActGelu) {
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = gelu(v[i]);
  }
  return v;
}

// Store of 4 finished values to C[m][n .. n+3] in the output type.  `vec`:
// n + 3 < N and N % 4 == 0 (one 16- or 8-byte store); otherwise the columns
// below N are stored one by one.  NT: non-temporal stores.
template <bool NT>
__device__ __forceinline__ void epi_put4(Epi e, int64_t N, int64_t m, int n, v4f v, bool vec) {
  if (e.out == kOutF32) {
    float* row = reinterpret_cast<float*>(e.C) + m * N;
    if (vec) {
      if (NT)
        __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(row + n));
      else
        *reinterpret_cast<v4f*>(row + n) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (n + i < N) row[n + i] = v[i];
    }
    return;
  }
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; i++) h[i] = e.out == kOutBF16 ? bf16_bits(v[i]) : f16_bits(v[i]);
  uint16_t* row = reinterpret_cast<uint16_t*>(e.C) + m * N;
  if (vec) {
    const v2i p = {(int)(h[0] | (h[1] << 16)), (int)(h[2] | (h[3] << 16))};
    if (NT)
      __builtin_nontemporal_store(p, reinterpret_cast<v2i*>(row + n));
    else
      *reinterpret_cast<v2i*>(row + n) = p;
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (n + i < N) row[n + i] = (uint16_t)h[i];
  }
}

template <bool NT>
__device__ __forceinline__ void epi_store4(Epi e, int64_t N, int64_t m, int n, v4f v, bool vec) {
  epi_put4<NT>(e, N, m, n, epi_apply(e, N, n, v, vec), vec);
}

}  // namespace mxg
