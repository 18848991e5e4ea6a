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
typedef int v6i __attribute__((ext_vector_type(6)));  // an FP6 MFMA operand (6 registers)
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) void lds_void;

// MFMA operand-format ids (cbsz / blgp fields): E4M3, E5M2, E2M1.
constexpr int kFmtFp8 = 0;
constexpr int kFmtBf8 = 1;
constexpr int kFmtFp4 = 4;
// FP6 element formats (E2M3 and E3M2: the format ids the scaled MFMA gives
// them).  An FP6 operand is 6 registers per lane: 32 codes of 6 bits,
// element i of the lane at bits 6i .. 6i+5.
constexpr int kFmtFp6 = 2;
constexpr int kFmtBf6 = 3;
// Integer element formats (not MFMA formats: remapped onto E4M3 / E2M1
// operand codes, see int4x8_to_e4m3 / int2x16_to_e2m1).
constexpr int kElemInt4 = 8;
constexpr int kElemInt2 = 9;

// XOR swizzle of the 16-byte chunk index inside an LDS row.  Fragment reads
// have 16 consecutive lanes read 16 consecutive rows at the same logical
// chunk; without a swizzle they conflict 3-way on gfx950.  The swizzle was
// chosen by measurement on MI355X (ds_read_b128 throughput and the
// SQ_LDS_BANK_CONFLICT counter): (row >> 1) & 7 and row & 7 are
// conflict-free, while (row ^ (row >> 3)) & 7 still conflicts 2-way.  Tile
// copies write LDS linearly (1 KiB per wave instruction) whatever the
// swizzle, because the swizzle is applied to the global source address.
// Rows of 8 chunks (128 bytes): fp8 and fp16 operands.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }
// Rows of 4 chunks (64 bytes): packed fp4 operands.
__device__ __forceinline__ int swz4(int row) { return (row >> 1) & 3; }

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

// ---- integer weights: lossless remap onto scaled-MFMA operand codes -------
//
// Two's complement INT4 values -8..7 are exact E4M3 values and INT2 values
// -2..1 are exact E2M1 values, so an integer operand is fed to the scaled
// fp8 / fp4 MFMA by replacing every code with the float code of the same
// value (the UE8M0 block scales are unchanged): the products and therefore
// the results are those of the integer operand.  The lookups run on four
// bytes at a time with v_perm_b32, whose selector bytes 0-3 pick bytes of
// its second source and 4-7 bytes of its first; selector values above 7 give
// a constant byte instead: 8, 9, 10, 11 repeat bit 7 of source bytes 1, 3, 5
// and 7 eight times, 12 gives 0x00 and 13-15 give 0xFF.

// Byte-wise lookup of four 4-bit indices (one per byte, 0..15) in a 16-entry
// table held as two 8-byte halves that are XORed: the first half is indexed
// with n, the second with n ^ 8.  For n < 8 the first permute returns a table
// byte and the second one of the constant bytes above (n ^ 8 >= 8), and for
// n >= 8 the other way round, so each half stores the wanted byte XOR the
// constant byte that the other half returns for the same n.  That constant is
// known for every n (selectors 8-11 read bit 7 of the other half's odd
// bytes), and the halves can be filled one after the other with no circular
// dependence: it costs two permutes and two XORs per four bytes, against
// three permutes and a selector computation for a byte select.
__device__ __forceinline__ uint32_t lookup16x(uint32_t idx, uint32_t lo0, uint32_t lo1, uint32_t hi0, uint32_t hi1) {
  return __builtin_amdgcn_perm(lo1, lo0, idx) ^ __builtin_amdgcn_perm(hi1, hi0, idx ^ 0x08080808u);
}

// The nibbles 0-3 (lo) and 4-7 (hi) of x, one per byte (low nibble of each
// byte; the high nibble is cleared).
__device__ __forceinline__ void spread_nibbles(uint32_t x, uint32_t& lo, uint32_t& hi) {
  const uint32_t s = x >> 4;
  lo = __builtin_amdgcn_perm(s, x, 0x05010400u) & 0x0F0F0F0Fu;
  hi = __builtin_amdgcn_perm(s, x, 0x07030602u) & 0x0F0F0F0Fu;
}

// Eight INT4 codes (element i in bits 4i .. 4i+3) -> the E4M3 codes of
// elements 0-3 (lo) and 4-7 (hi), one per byte.
__device__ __forceinline__ void int4x8_to_e4m3(uint32_t x, uint32_t& lo, uint32_t& hi) {
  // E4M3 codes of 0..7 (n = 0..7) and of -8..-1 (n = 8..15):
  //   00 38 40 44 48 4A 4C 4E  D0 CE CC CA C8 C4 C0 B8
  // stored as described at lookup16x (bytes in index order, low byte first)
  constexpr uint32_t L0 = 0x444038FFu, L1 = 0xB1B3B548u, H0 = 0x3533CED0u, H1 = 0x473F3BC8u;
  uint32_t a, b;
  spread_nibbles(x, a, b);
  lo = lookup16x(a, L0, L1, H0, H1);
  hi = lookup16x(b, L0, L1, H0, H1);
}

// Sixteen INT2 codes (element i in bits 2i .. 2i+1) -> the E2M1 codes of
// elements 0-7 (lo) and 8-15 (hi), two per byte, even element in the low
// nibble.  A nibble of x holds a pair of INT2 codes p = c0 + 4 c1, and its
// table entry is the byte of their two E2M1 codes, code(c0) | code(c1) << 4,
// with code 0 -> 0x0, 1 -> 0x2 (1.0), -2 -> 0xC, -1 -> 0xA:
//   00 02 0C 0A 20 22 2C 2A  C0 C2 CC CA A0 A2 AC AA
__device__ __forceinline__ void int2x16_to_e2m1(uint32_t x, uint32_t& lo, uint32_t& hi) {
  constexpr uint32_t L0 = 0x0A0C02FFu, L1 = 0xD5D3DD20u, H0 = 0x3533C2C0u, H1 = 0x55535DA0u;
  uint32_t a, b;
  spread_nibbles(x, a, b);
  lo = lookup16x(a, L0, L1, H0, H1);
  hi = lookup16x(b, L0, L1, H0, H1);
}

// The format ids must be compile-time constants for the builtin.
template <int FA, int FB>
__device__ __forceinline__ v4f mfma_scaled_16x16x128(const v8i& a, const v8i& b, const v4f& c, int scale_a,
                                                      int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FA, FB, 0, scale_a, 0, scale_b);
}

// Scaled MFMA with the accumulator tied in place (dst == srcC, AGPRs).  The
// builtin form lets the register allocator pick dst != srcC for this
// instruction, which on this compiler adds accumulator copies and hazard
// NOPs inside the K loop and halves the MFMA issue rate (measured: 16 chained
// accumulators reach ~4.5 PFLOP/s tied versus ~2.5 in the K loop with the
// builtin).  The hardware interlocks on the srcA/srcB/scale VGPRs written by
// LDS loads through the waitcnt the compiler inserts for the asm operands;
// accumulators are only touched by these instructions until mfma_drain().
template <int FA, int FB>
__device__ __forceinline__ void mfma_scaled_acc(v4f& c, const v8i& a, const v8i& b, int scale_a, int scale_b) {
  if constexpr (FA == kFmtFp8 && FB == kFmtFp8) {
    asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
        : "+a"(c) : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b));
  } else if constexpr ((FA == kFmtFp6 || FA == kFmtBf6) && FB == kFmtFp8) {
    // an FP6 first operand takes 6 registers (32 six-bit codes per lane);
    // the compiler gathers them with VALU moves just before this MFMA and
    // inserts no wait states for an inline MFMA's operands: the s_nop does
    const v6i a6 = {a[0], a[1], a[2], a[3], a[4], a[5]};
    asm("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:%5"
        : "+a"(c) : "v"(a6), "v"(b), "v"(scale_a), "v"(scale_b), "i"(FA));
  } else if constexpr (FA != kFmtFp4 && FB != kFmtFp4) {
    // 8-register operands with an E5M2 side: the format ids go in cbsz / blgp
    asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:%5 blgp:%6"
        : "+a"(c) : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b), "i"(FA), "i"(FB));
  } else if constexpr (FA == kFmtFp4 && FB == kFmtFp8) {
    const v4i a4 = {a[0], a[1], a[2], a[3]};
    asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4"
        : "+a"(c) : "v"(a4), "v"(b), "v"(scale_a), "v"(scale_b));
  } else if constexpr (FA == kFmtFp8 && FB == kFmtFp4) {
    const v4i b4 = {b[0], b[1], b[2], b[3]};
    asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] blgp:4"
        : "+a"(c) : "v"(a), "v"(b4), "v"(scale_a), "v"(scale_b));
  } else {
    static_assert(FA == kFmtFp4 && FB == kFmtFp4, "fp4 pairs only with E4M3 or E2M1");
    const v4i a4 = {a[0], a[1], a[2], a[3]};
    const v4i b4 = {b[0], b[1], b[2], b[3]};
    asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4 blgp:4"
        : "+a"(c) : "v"(a4), "v"(b4), "v"(scale_a), "v"(scale_b));
  }
}

// E4M3 x E4M3 scaled MFMA (accumulator tied as above) whose operand a VALU
// instruction may have written just before (codes remapped in registers):
// the compiler inserts no wait states for an inline MFMA's operands, so the
// s_nop supplies them.
__device__ __forceinline__ void mfma_scaled_acc_after_valu(v4f& c, const v8i& a, const v8i& b, int scale_a,
                                                           int scale_b) {
  asm("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
      : "+a"(c) : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b));
}

// The same for an E2M1 first operand (remapped codes) against an E4M3
// second one.
__device__ __forceinline__ void mfma_scaled_acc_fp4a_after_valu(v4f& c, const v8i& a, const v8i& b, int scale_a,
                                                                int scale_b) {
  const v4i a4 = {a[0], a[1], a[2], a[3]};
  asm("s_nop 4\n\tv_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:4"
      : "+a"(c) : "v"(a4), "v"(b), "v"(scale_a), "v"(scale_b));
}

// Scaled MFMA taking its scales from byte BA of scale_a and byte BB of
// scale_b (the op_sel / op_sel_hi pair selects the byte), so that the scales
// of four fragments share one VGPR.  Accumulator tied as above; volatile, so
// the MFMAs keep program order with respect to other volatile asm (barriers,
// waits) and stay inside the phase that issues them.
template <int FA, int FB, int BA, int BB>
__device__ __forceinline__ void mfma_scaled_acc_pk(v4f& c, const v8i& a, const v8i& b, int scale_a, int scale_b) {
  static_assert(BA >= 0 && BA < 4 && BB >= 0 && BB < 4, "scale byte index");
  if constexpr (FA == kFmtFp8 && FB == kFmtFp8) {
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0]"
                 : "+a"(c)
                 : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b), "i"(BA & 1), "i"(BB & 1), "i"(BA >> 1), "i"(BB >> 1));
  } else if constexpr (FA != kFmtFp4 && FB != kFmtFp4) {
    asm volatile(
        "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0] cbsz:%9 "
        "blgp:%10"
        : "+a"(c)
        : "v"(a), "v"(b), "v"(scale_a), "v"(scale_b), "i"(BA & 1), "i"(BB & 1), "i"(BA >> 1), "i"(BB >> 1), "i"(FA),
          "i"(FB));
  } else if constexpr (FA == kFmtFp4 && FB == kFmtFp8) {
    const v4i a4 = {a[0], a[1], a[2], a[3]};
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0] cbsz:4"
                 : "+a"(c)
                 : "v"(a4), "v"(b), "v"(scale_a), "v"(scale_b), "i"(BA & 1), "i"(BB & 1), "i"(BA >> 1), "i"(BB >> 1));
  } else if constexpr (FA == kFmtFp8 && FB == kFmtFp4) {
    const v4i b4 = {b[0], b[1], b[2], b[3]};
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0] blgp:4"
                 : "+a"(c)
                 : "v"(a), "v"(b4), "v"(scale_a), "v"(scale_b), "i"(BA & 1), "i"(BB & 1), "i"(BA >> 1), "i"(BB >> 1));
  } else {
    static_assert(FA == kFmtFp4 && FB == kFmtFp4, "fp4 pairs only with E4M3 or E2M1");
    const v4i a4 = {a[0], a[1], a[2], a[3]};
    const v4i b4 = {b[0], b[1], b[2], b[3]};
    asm volatile(
        "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[%5,%6,0] op_sel_hi:[%7,%8,0] cbsz:4 blgp:4"
        : "+a"(c)
        : "v"(a4), "v"(b4), "v"(scale_a), "v"(scale_b), "i"(BA & 1), "i"(BB & 1), "i"(BA >> 1), "i"(BB >> 1));
  }
}
// fp16 16x16x32 MFMA, accumulator tied in AGPRs; a and b hold 8 halves each.
__device__ __forceinline__ void mfma_f16_acc_v(v4f& c, const v4i& a, const v4i& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Wait states between the last MFMA writing an accumulator and any other
// instruction reading it (the compiler does not model the inline MFMA's
// latency): 3 x 16 idle cycles cover the 16-pass worst case; the empty asm
// ties every accumulator to this point so no read is scheduled above it.
template <int NI, int NJ>
__device__ __forceinline__ void mfma_drain(v4f (&acc)[NI][NJ]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < NI; i++)
#pragma unroll
    for (int j = 0; j < NJ; j++) asm volatile("" : "+a"(acc[i][j]));
}
// Wait states between writing the accumulators' initial zeros and the first
// inline MFMA reading them.
template <int NI, int NJ>
__device__ __forceinline__ void mfma_fence_init(v4f (&acc)[NI][NJ]) {
#pragma unroll
  for (int i = 0; i < NI; i++)
#pragma unroll
    for (int j = 0; j < NJ; j++) asm volatile("" : "+a"(acc[i][j]));
  asm volatile("s_nop 7" ::: "memory");
}

__device__ __forceinline__ v4f mfma_f16_16x16x32(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

}  // namespace mxg
