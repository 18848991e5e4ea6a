// mxg_internal.h - host-side launchers behind the C ABI (not exported).
// Every launcher assumes validated arguments and enqueues on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxg_epilogue.h"

namespace mxg {

hipError_t launch_quantize(const float* X, int64_t rows, int64_t K, int elem, void* Q, uint8_t* S,
                           hipStream_t stream);

// fmt: 0 = E4M3 x E4M3, 1 = E4M3 x E2M1, 2 = E2M1 x E2M1, 3 = E5M2 x E5M2,
// 4 = E4M3 x E5M2, 5 = E5M2 x E4M3, 6 = E4M3 x INT4, 7 = E4M3 x INT2 (A x B).  The MX launchers write
// C through the epilogue `e` (output pointer, bias, activation, output type).
hipError_t launch_mx_tiled(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                           int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream);
// Split-K skinny kernel (M <= kSkinnyMaxM, fmt 0, 1, 6 or 7) over the k range
// [k0, k0 + kn) of a product whose rows hold K elements (kn < 0: to K).  With
// k0 > 0, C is fp32 and already holds the sum over k < k0, which is added.
hipError_t launch_mx_skinny(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                            int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream, int64_t k0 = 0,
                            int64_t kn = -1);
hipError_t launch_f16_tiled(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N, int64_t K,
                            int b_is_nk, hipStream_t stream);
hipError_t launch_deq_tiled(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, float* C, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream);

// 8-wave ping-pong kernels for full 256 x 256 tiles (M, N multiples of 256;
// MX: K % 128 == 0 and 4-byte aligned scale planes; fp16: K % 64 == 0 and an
// N x K right operand).
bool pingpong_mx_ok(const uint8_t* SA, const uint8_t* SB, int64_t M, int64_t N, int64_t K);
hipError_t launch_mx_pingpong(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                              int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream);
hipError_t launch_f16_pingpong(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream);
// The same ping-pong on 128 x 128 tiles with K split between the two wave
// groups (M, N multiples of 128; MX: K % 128 == 0 and 4-byte aligned scale
// planes; fp16: K % 64 == 0 and an N x K right operand).
bool pp128_mx_ok(const uint8_t* SA, const uint8_t* SB, int64_t M, int64_t N, int64_t K);
hipError_t launch_mx_pp128(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                           int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream);
hipError_t launch_f16_pp128(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream);

// Decode kernel for M <= 64 (MX fp8 x fp8 or fp8 x fp4): K a multiple of
// 1024 from 2048 (A's k range per wave is held in registers, which bounds one
// launch's K; longer K runs in chunks that add into an fp32 C), 4-byte
// aligned scale planes.
// launch_mx_decode covers k < kn of rows that hold K elements (kn < 0: all
// of K; kn a multiple of 1024 that decode_ok(M, kn, ...) accepts).
bool decode_ok(int64_t M, int64_t K, int fmt, const uint8_t* SA, const uint8_t* SB, const Epi& e);
hipError_t launch_mx_decode(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                            int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream, int64_t kn = -1);

// Stand-alone epilogue: Y = out(act(X + bias)) for an M x N fp32 matrix X,
// written through `e` (the decomposed form of the fused GEMM epilogue).
hipError_t launch_epilogue(const float* X, int64_t M, int64_t N, const Epi& e, hipStream_t stream);

// Largest M served by the split-K streaming kernel.
constexpr int64_t kSkinnyMaxM = 64;

}  // namespace mxg
