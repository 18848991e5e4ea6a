// mxg_device.h - device-side building blocks shared by the gfx950 kernels:
// vector types, LDS swizzles, direct global->LDS copies, the workgroup ->
// output-tile map and the MFMA operand layouts.
//
// Operand register layouts of the CDNA4 16x16 MFMA family, as measured on
// MI355X with one-hot and random operands (lane l, g = l / 16, r = l % 16):
//   scaled fp8 operand (32 bytes, 8 VGPRs):   row r; bytes 0..15 hold
//       k = 16g .. 16g+15, bytes 16..31 hold k = 64+16g .. 64+16g+15
//   scaled fp4 operand (16 bytes, 4 VGPRs):   row r; nibbles 0..31 hold
//       k = 32g .. 32g+31, even k in the low nibble
//   scale operand (one byte of a VGPR, chosen by op_sel): row r, 32-element
//       block g of the 128-element step
//   fp16 16x16x32 operand (8 halves):          row r; k = 8g .. 8g+7
//   16x16 fp32 result (4 VGPRs):               D[4g + i][r], i = 0..3, where
//       the D row comes from the first source operand's rows and the D
//       column from the second source operand's rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) void lds_void;

// MFMA operand-format ids (cbsz / blgp fields).
constexpr int kFmtFp8 = 0;
constexpr int kFmtFp4 = 4;

// XOR swizzle of the 16-byte chunk index inside an LDS row, chosen so that
// the fragment reads (16 consecutive lanes = 16 consecutive rows, same
// logical chunk) and the row-major tile writes hit distinct banks both when
// 8 lanes and when 16 lanes are served per LDS cycle.
// Rows of 8 chunks (128 bytes): fp8 and fp16 operands.
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }
// Rows of 4 chunks (64 bytes): packed fp4 operands.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

// Direct global -> LDS copy of 16 bytes per lane.  The LDS destination of
// lane i is lds_base + 16 * i; lds_base must be wave-uniform.
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_base, 16, 0, 0);
}

// Workgroup id -> (tile_m, tile_n).  Consecutive workgroup ids are dispatched
// round-robin over the 8 XCDs, each with its own L2; the first step gives
// every XCD a contiguous range of tile ids.  The second step walks that range
// in groups of kGroupM tile rows so that concurrently running workgroups of
// one XCD share A rows and B columns in that XCD's L2.
__device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int id = bid;
  if ((total & 7) == 0) id = (bid & 7) * (total >> 3) + (bid >> 3);
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * tiles_n;
  const int group = id / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  const int in = id - group * per_group;
  tm = first_m + in % gsz;
  tn = in / gsz;
}

// The format ids must be compile-time constants for the builtin.
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_scaled_16x16x128(const v8i& a, const v8i& b, const v4f& c, int scale_a,
                                                      int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, scale_a, 0, scale_b);
}

__device__ __forceinline__ v4f mfma_f16_16x16x32(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace mxg
