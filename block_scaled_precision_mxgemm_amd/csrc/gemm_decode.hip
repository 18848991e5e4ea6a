// gemm_decode.hip - MX GEMM for decode shapes with at most 16 activation rows
// (M <= 16) against a large weight matrix B (N x K, MXFP8 or MXFP4).  The
// product is bound by the bytes of B, which must stream from HBM exactly
// once; the weight plane is what quantization shrinks ("Metal tensors で
// カスタム機械学習オペレーションを最適化する", section "主要内容": inference
// is memory-bandwidth bound and quantization cuts both the footprint and the
// traffic).
//
// Design (gfx950):
//   * one persistent workgroup of 8 waves per CU owns a contiguous range of
//     16-row blocks of B ("fragments") and streams them through LDS in
//     stages of 16 rows x 1 KiB (a quarter row for the 8192-wide fp4 weights)
//     with direct global->LDS copies.  Each copy instruction reads one row's
//     contiguous 1 KiB, the access pattern that measured fastest on MI355X
//     (5.8 TB/s for a 112 MiB read, against 4.3 TB/s when every instruction
//     takes 64 bytes from each of 16 rows);
//   * inside a stage row the 16-byte chunks are XOR-swizzled with the row
//     index (applied on the global side, so the copy still writes LDS
//     linearly), which makes the MFMA fragment reads conflict-free;
//   * a ring of kDecStages stages keeps the copies of the next stages in
//     flight while the current one is multiplied; one barrier per stage;
//   * every wave takes 1/8 of each stage's MFMAs (2 for fp4, 1 for fp8) and
//     holds the matching k range of A (16 rows) in registers for the whole
//     kernel;
//   * a fragment's 8 per-wave partial sums go to LDS and one wave adds them
//     in a fixed order one stage later, so the result is deterministic and
//     needs no atomics.
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

constexpr int kDecWaves = 8;
constexpr int kDecStages = 7;
constexpr int kStageRowBytes = 1024;  // bytes of one B row per stage

struct DecArgs {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  float* C;
  int M, N, K;
  int nfrags;  // ceil(N / 16)
};

// Wait until this wave has at most 15 (steady state: the copies of the
// kDecStages - 2 younger stages, 3 per stage) or 0 global->LDS copies in
// flight; the count is an immediate.
__device__ __forceinline__ void wait_copies(bool all) {
  if (all)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
}
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool BF4, int KA>
struct Decode {
  static constexpr int MPW = BF4 ? 2 : 1;          // MFMAs per wave per stage
  static constexpr int MPS = MPW * kDecWaves;      // MFMAs per stage (128 k each)
  static constexpr int NQ = KA / MPW;              // stages per fragment
  static constexpr int SROW = BF4 ? 64 : 32;       // scale bytes per row per stage
  static constexpr int SZ_ST = 16 * kStageRowBytes;
  static constexpr int SZ_SC = 16 * SROW;
  static constexpr int OFF_ST = 0;
  static constexpr int OFF_SC = OFF_ST + kDecStages * SZ_ST;
  static constexpr int OFF_PART = OFF_SC + kDecStages * SZ_SC;
  static constexpr int LDS = OFF_PART + 2 * kDecWaves * 64 * 16;
  static_assert(LDS <= 160 * 1024, "fits the 160 KiB LDS of a gfx950 CU");
  static_assert(NQ >= 1 && KA % MPW == 0, "whole stages per fragment");
  static_assert(3 * (kDecStages - 2) == 15, "wait_copies immediate");

  // fp8 operand of the MFMA covering k0 .. k0+127 of row `p` (p at k0):
  // lane group g holds k0 + 16g .. +15 and k0 + 64 + 16g .. +15
  static __device__ __forceinline__ v8i load_fp8_op(const uint8_t* p, int g) {
    const v4i lo = *reinterpret_cast<const v4i*>(p + 16 * g);
    const v4i hi = *reinterpret_cast<const v4i*>(p + 64 + 16 * g);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }

  static __device__ __forceinline__ void reduce_store(const DecArgs& a, const uint8_t* smem, int frag, int slot,
                                                      int lane, int g, int r) {
    const v4f* part = reinterpret_cast<const v4f*>(smem + OFF_PART) + (size_t)slot * kDecWaves * 64;
    v4f s = part[lane];
#pragma unroll
    for (int w = 1; w < kDecWaves; w++) s += part[w * 64 + lane];
    // lane (g, r) holds C[r][16 frag + 4g .. 4g+3]
    const int m = r;
    const int n = frag * 16 + 4 * g;
    if (m < a.M) {
      float* crow = a.C + (int64_t)m * a.N;
      if ((a.N & 3) == 0 && n + 3 < a.N) {
        *reinterpret_cast<v4f*>(crow + n) = s;
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (n + i < a.N) crow[n + i] = s[i];
      }
    }
  }

  static __device__ __forceinline__ void run(const DecArgs& a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    // balanced contiguous split of the fragments over the workgroups
    const int f_begin = (int)((int64_t)a.nfrags * blockIdx.x / gridDim.x);
    const int nf = (int)((int64_t)a.nfrags * (blockIdx.x + 1) / gridDim.x) - f_begin;
    const int S = nf * NQ;  // stages of this workgroup
    const uint32_t rb = BF4 ? (uint32_t)(a.K >> 1) : (uint32_t)a.K;  // bytes per B row
    const uint32_t nb = (uint32_t)(a.K >> 5);                         // scale bytes per row

    // Copies: wave w fetches stage rows 2w and 2w+1 (lane l writes physical
    // chunk l of the row and fetches logical chunk l ^ (row & 15)) and the
    // scale bytes of the same two rows, 4 bytes per lane on the first
    // 2 * SROW / 4 lanes (global->LDS copies of fewer than 4 bytes still
    // write one dword per lane).  Every wave issues exactly 3 copies per
    // stage, which the wait counts rely on.
    constexpr int kRsrcWord3 = 0x00020000;
    constexpr int SL = SROW / 4;  // scale lanes per row
    const uint32_t vo0 = (uint32_t)((lane ^ ((2 * wave) & 15)) * 16);
    const uint32_t vo1 = (uint32_t)((lane ^ ((2 * wave + 1) & 15)) * 16);
    const int srow_l = 2 * wave + (lane / SL) % 2;  // scale row of this lane
    const uint32_t sbyte_l = (uint32_t)((lane % SL) * 4);
    auto issue = [&](int s) {
      const int f = s / NQ, q = s - f * NQ, buf = s % kDecStages;
      const int row0 = (f_begin + f) * 16;
      const auto rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)(a.B + (int64_t)row0 * rb), 0, 16 * rb, kRsrcWord3);
      const auto rs_s = __builtin_amdgcn_make_buffer_rsrc((void*)(a.SB + (int64_t)row0 * nb), 0, 16 * nb, kRsrcWord3);
      uint8_t* st = smem + OFF_ST + buf * SZ_ST;
      const int r0 = min(row0 + 2 * wave, a.N - 1) - row0;  // rows past N: the last row again
      const int r1 = min(row0 + 2 * wave + 1, a.N - 1) - row0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(st + (2 * wave) * kStageRowBytes), 16, vo0,
                                               (uint32_t)r0 * rb + (uint32_t)q * kStageRowBytes, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(st + (2 * wave + 1) * kStageRowBytes), 16, vo1,
                                               (uint32_t)r1 * rb + (uint32_t)q * kStageRowBytes, 0, 0);
      const uint32_t sr = (uint32_t)(min(row0 + srow_l, a.N - 1) - row0);
      if (lane < 2 * SL)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (lds_void*)(smem + OFF_SC + buf * SZ_SC + wave * 2 * SROW), 4,
                                                 sr * nb + sbyte_l, (uint32_t)q * SROW, 0, 0);
    };

    // Prologue: stage 0, then A, then stages 1 .. kDecStages-2.  The vector
    // memory counter completes in issue order, so waiting for stage 0 and A
    // at the first stage leaves the younger stages in flight.
    if (S > 0) issue(0);

    // A (rows clamped to M-1; rows >= M are computed and discarded): the k
    // ranges of this wave's MFMAs, stage q, local MFMA t -> global MFMA
    // j = q * MPS + wave * MPW + t; its scale is the byte of block 4j + g
    v8i av[KA];
    int sa[KA];
    {
      const int m = min(r, a.M - 1);
      const uint8_t* row = a.A + (int64_t)m * a.K;
      const uint8_t* srow = a.SA + (int64_t)m * nb;
#pragma unroll
      for (int q = 0; q < NQ; q++)
#pragma unroll
        for (int t = 0; t < MPW; t++) {
          const int j = q * MPS + wave * MPW + t;
          av[q * MPW + t] = load_fp8_op(row + (int64_t)j * 128, g);
          const uint32_t s4 = *reinterpret_cast<const uint32_t*>(srow + 4 * j);
          sa[q * MPW + t] = (int)__builtin_amdgcn_ubfe(s4, 8 * g, 8);
        }
    }

#pragma unroll
    for (int s = 1; s < kDecStages - 1; s++)
      if (s < S) issue(s);

    v4f acc[MPW];
#pragma unroll
    for (int t = 0; t < MPW; t++) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    // stage s = f * NQ + q; the q loop is unrolled so that A and its scales
    // stay in registers (a runtime index would put them in scratch memory)
    for (int f = 0; f < nf; f++) {
#pragma unroll
      for (int q = 0; q < NQ; q++) {
        const int s = f * NQ + q, buf = s % kDecStages;
        // This wave's copies of stage s are done once at most the younger
        // stages' copies are in flight (all of them near the end, where
        // fewer younger stages were issued); the barrier publishes every
        // wave's.
        wait_copies(s + kDecStages - 2 > S - 1);
        stage_barrier();
        if (s + kDecStages - 1 < S) issue(s + kDecStages - 1);  // into the buffer read at stage s-1
        // the previous fragment's partials were published by the barrier
        if (q == 0 && f > 0 && wave == (f - 1) % kDecWaves)
          reduce_store(a, smem, f_begin + f - 1, (f - 1) & 1, lane, g, r);
        const uint8_t* st = smem + OFF_ST + buf * SZ_ST;
        const uint8_t* sc = smem + OFF_SC + buf * SZ_SC;
#pragma unroll
        for (int t = 0; t < MPW; t++) {
          const int lj = wave * MPW + t;  // MFMA index inside the stage
          v8i bv;
          if (BF4) {
            const int ch = (lj * 4 + g) ^ r;  // 16-byte chunk, swizzled
            const v4i lo = *reinterpret_cast<const v4i*>(st + r * kStageRowBytes + ch * 16);
            bv = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
          } else {
            const int cl = (lj * 8 + g) ^ r, chh = (lj * 8 + 4 + g) ^ r;
            const v4i lo = *reinterpret_cast<const v4i*>(st + r * kStageRowBytes + cl * 16);
            const v4i hi = *reinterpret_cast<const v4i*>(st + r * kStageRowBytes + chh * 16);
            bv = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          const int sb = sc[r * SROW + lj * 4 + g];
          acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, av[q * MPW + t], acc[t],
                                                                    BF4 ? kFmtFp4 : kFmtFp8, kFmtFp8, 0, sb, 0,
                                                                    sa[q * MPW + t]);
        }
      }
      v4f p = acc[0];
#pragma unroll
      for (int t = 1; t < MPW; t++) p += acc[t];
      reinterpret_cast<v4f*>(smem + OFF_PART)[((f & 1) * kDecWaves + wave) * 64 + lane] = p;
#pragma unroll
      for (int t = 0; t < MPW; t++) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    stage_barrier();
    if (nf > 0 && wave == (nf - 1) % kDecWaves) reduce_store(a, smem, f_begin + nf - 1, (nf - 1) & 1, lane, g, r);
  }
};

template <bool BF4, int KA>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512))) void decode_kernel(DecArgs a) {
  Decode<BF4, KA>::run(a);
}

template <bool BF4, int KA>
hipError_t launch_dec(const DecArgs& a, int cus, hipStream_t stream) {
  const int grid = a.nfrags < cus ? a.nfrags : cus;
  hipLaunchKernelGGL((decode_kernel<BF4, KA>), dim3(grid), dim3(kDecWaves * 64), 0, stream, a);
  return hipGetLastError();
}

template <bool BF4>
hipError_t launch_dec_k(const DecArgs& a, int cus, hipStream_t stream) {
  switch (a.K) {
    case 2048: return launch_dec<BF4, 2>(a, cus, stream);
    case 4096: return launch_dec<BF4, 4>(a, cus, stream);
    default: return launch_dec<BF4, 8>(a, cus, stream);
  }
}

}  // namespace

bool decode_ok(int64_t M, int64_t K, int fmt, const uint8_t* SA, const uint8_t* SB) {
  return M <= 16 && (fmt == 0 || fmt == 1) && (K == 2048 || K == 4096 || K == 8192) &&
         (((uintptr_t)SA | (uintptr_t)SB) & 3) == 0;
}

hipError_t launch_mx_decode(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, float* C, int64_t M,
                            int64_t N, int64_t K, int fmt, hipStream_t stream) {
  DecArgs a{};
  a.A = (const uint8_t*)A;
  a.SA = SA;
  a.B = (const uint8_t*)B;
  a.SB = SB;
  a.C = C;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.nfrags = (int)((N + 15) / 16);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus <= 0) cus = 1;
  return fmt == 1 ? launch_dec_k<true>(a, cus, stream) : launch_dec_k<false>(a, cus, stream);
}

}  // namespace mxg
