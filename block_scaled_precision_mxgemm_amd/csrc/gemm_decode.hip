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
#include <utility>

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

__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool BF4, int KA>
struct Decode {
  static constexpr int MPW = BF4 ? 2 : 1;          // MFMAs per wave per stage
  static constexpr int MPS = MPW * kDecWaves;      // MFMAs per stage (128 k each)
  static constexpr int NQ = KA / MPW;              // stages per fragment
  static constexpr int SROW = BF4 ? 64 : 32;       // scale bytes per row per stage
  static constexpr int SZ_ST = 16 * kStageRowBytes;
  static constexpr int SC_WAVE = 256;               // scale slot per wave per stage (64 lanes x 4 B)
  static constexpr int SZ_SC = kDecWaves * SC_WAVE;
  static constexpr int OFF_ST = 0;
  static constexpr int OFF_SC = OFF_ST + kDecStages * SZ_ST;
  static constexpr int OFF_PART = OFF_SC + kDecStages * SZ_SC;
  static constexpr int LDS = OFF_PART + 2 * kDecWaves * 64 * 16;
  static_assert(LDS <= 160 * 1024, "fits the 160 KiB LDS of a gfx950 CU");
  static_assert(NQ >= 1 && KA % MPW == 0, "whole stages per fragment");

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

  // Per-workgroup state shared by the stage functions (all in registers
  // once inlined).
  struct State {
    const DecArgs* a;
    uint8_t* smem;
    int lane, wave, g, r;
    int f_begin, nf, S;
    uint32_t rb, nb;  // bytes per B row, scale bytes per row
    uint32_t vo0, vo1, sbyte_l;
    int srow_l;
    v8i av[KA];   // A operands of this wave's MFMAs
    uint32_t sa[KA];  // their scale dwords (blocks 4j .. 4j+3); byte g is extracted at the MFMA
    v4f acc[MPW];
  };

  // Vector-memory instructions per A load group (stage q of the A registers):
  // lo and hi 16-byte halves per MFMA plus one load of the MPW scale dwords.
  static constexpr int LA = 2 * MPW + 1;
  static constexpr int kYoung = 3 * (kDecStages - 2);  // copies of the younger stages in flight

  template <int N>
  static __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
  }
  static __device__ __forceinline__ void order_fence() { asm volatile("" ::: "memory"); }

  // Copies of stage s: wave w fetches stage rows 2w and 2w+1 (lane l writes
  // physical chunk l of the row and fetches logical chunk l ^ (row & 15)) and
  // the scale bytes of the same two rows into its own 256-byte slot, 4 bytes
  // per lane (global->LDS copies of fewer than 4 bytes still write one dword
  // per lane): row 2w at slot byte 0, row 2w+1 at SROW; the remaining lanes
  // fetch a valid address again into the slot's unused tail.  Every wave
  // issues exactly 3 copies per stage, all lanes active, which the wait
  // counts rely on (a copy under a lane condition could be skipped, and the
  // compiler would then count conservatively).
  static __device__ __forceinline__ void issue(State& t, int s) {
    constexpr int kRsrcWord3 = 0x00020000;
    const DecArgs& a = *t.a;
    // past the workgroup's last stage, that stage's source again: the copy
    // lands in a buffer no real stage still needs, and the copy count per
    // stage stays fixed
    const int buf = s % kDecStages;
    const int sv = min(s, t.S - 1);
    const int f = sv / NQ, q = sv - f * NQ;
    const int row0 = (t.f_begin + f) * 16;
    const auto rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)(a.B + (int64_t)row0 * t.rb), 0, 16 * t.rb, kRsrcWord3);
    const auto rs_s = __builtin_amdgcn_make_buffer_rsrc((void*)(a.SB + (int64_t)row0 * t.nb), 0, 16 * t.nb, kRsrcWord3);
    uint8_t* st = t.smem + OFF_ST + buf * SZ_ST;
    const int r0 = min(row0 + 2 * t.wave, a.N - 1) - row0;  // rows past N: the last row again
    const int r1 = min(row0 + 2 * t.wave + 1, a.N - 1) - row0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(st + (2 * t.wave) * kStageRowBytes), 16, t.vo0,
                                             (uint32_t)r0 * t.rb + (uint32_t)q * kStageRowBytes, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(st + (2 * t.wave + 1) * kStageRowBytes), 16, t.vo1,
                                             (uint32_t)r1 * t.rb + (uint32_t)q * kStageRowBytes, 0, 0);
    const uint32_t sr = (uint32_t)(min(row0 + t.srow_l, a.N - 1) - row0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (lds_void*)(t.smem + OFF_SC + buf * SZ_SC + t.wave * SC_WAVE), 4,
                                             sr * t.nb + t.sbyte_l, (uint32_t)q * SROW, 0, 0);
  }

  // A for the stage-q MFMAs of this wave (rows clamped to M-1; rows >= M are
  // computed and discarded): local MFMA u -> global MFMA j = q * MPS +
  // wave * MPW + u covering k 128j .. 128j+127; its scale is byte g of the
  // dword of blocks 4j .. 4j+3.
  template <int Q>
  static __device__ __forceinline__ void load_a(State& t) {
    const DecArgs& a = *t.a;
    const int m = min(t.r, a.M - 1);
    const uint8_t* row = a.A + (int64_t)m * a.K;
    const uint8_t* srow = a.SA + (int64_t)m * t.nb;
    const int j0 = Q * MPS + t.wave * MPW;
#pragma unroll
    for (int u = 0; u < MPW; u++) t.av[Q * MPW + u] = load_fp8_op(row + (int64_t)(j0 + u) * 128, t.g);
    // the scale dwords stay raw until the MFMA: extracting the byte here would
    // wait for this load in the middle of the prologue
    if constexpr (MPW == 2) {
      const v2i d = *reinterpret_cast<const v2i*>(srow + 4 * j0);  // one 8-byte load
      t.sa[Q * MPW] = (uint32_t)d[0];
      t.sa[Q * MPW + MPW - 1] = (uint32_t)d[1];
    } else {
      t.sa[Q * MPW] = *reinterpret_cast<const uint32_t*>(srow + 4 * j0);
    }
  }

  // Prologue, in this issue order: stage p's copies then A(p), for p = 0 ..;
  // stages up to kDecStages - 2, A up to NQ - 1.
  template <int... P>
  static __device__ __forceinline__ void prologue(State& t, std::integer_sequence<int, P...>) {
    (
        [&] {
          if (P < kDecStages - 1) issue(t, P);
          order_fence();
          if constexpr (P < NQ) load_a<P>(t);
          order_fence();
        }(),
        ...);
  }

  // Stage q of fragment f (s = f * NQ + q).
  template <int Q, bool FIRST>
  static __device__ __forceinline__ void stage(State& t, int f) {
    const DecArgs& a = *t.a;
    const int s = f * NQ + Q, buf = s % kDecStages;
    // This wave's copies of stage s are complete once at most the younger
    // vector-memory instructions are outstanding (the counter completes in
    // issue order).  Younger than stage s's copies: the copies of the
    // kDecStages - 2 younger stages (always issued, see issue()) and, in the
    // first fragment, the A loads of stages q .. NQ-1 when stage q was a
    // prologue stage.  Stores of C issued since are younger still and only
    // make the wait stricter.
    if (FIRST && Q < kDecStages - 1)
      wait_vm<kYoung + (Q < kDecStages - 1 ? LA * (NQ - Q) : 0)>();
    else
      wait_vm<kYoung>();
    stage_barrier();                       // publishes every wave's copies of stage s
    issue(t, s + kDecStages - 1);          // into the buffer read at stage s-1
    // the previous fragment's partials were published by the barrier
    if (!FIRST && Q == 0 && t.wave == (f - 1) % kDecWaves)
      reduce_store(a, t.smem, t.f_begin + f - 1, (f - 1) & 1, t.lane, t.g, t.r);
    const uint8_t* st = t.smem + OFF_ST + buf * SZ_ST;
    const uint8_t* sc = t.smem + OFF_SC + buf * SZ_SC;
    const int g = t.g, r = t.r;
#pragma unroll
    for (int u = 0; u < MPW; u++) {
      const int lj = t.wave * MPW + u;  // MFMA index inside the stage
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
      const int sb = sc[(r >> 1) * SC_WAVE + (r & 1) * SROW + lj * 4 + g];
      t.acc[u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bv, t.av[Q * MPW + u], t.acc[u],
                                                                  BF4 ? kFmtFp4 : kFmtFp8, kFmtFp8, 0, sb, 0,
                                                                  (int)__builtin_amdgcn_ubfe(t.sa[Q * MPW + u], 8 * g, 8));
    }
  }

  template <bool FIRST, int... Q>
  static __device__ __forceinline__ void fragment(State& t, int f, std::integer_sequence<int, Q...>) {
    (stage<Q, FIRST>(t, f), ...);
    v4f p = t.acc[0];
#pragma unroll
    for (int u = 1; u < MPW; u++) p += t.acc[u];
    reinterpret_cast<v4f*>(t.smem + OFF_PART)[((f & 1) * kDecWaves + t.wave) * 64 + t.lane] = p;
#pragma unroll
    for (int u = 0; u < MPW; u++) t.acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  static __device__ __forceinline__ void run(const DecArgs& a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
    State t;
    t.a = &a;
    t.smem = smem;
    const int tid = threadIdx.x;
    t.lane = tid & 63;
    t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    t.g = t.lane >> 4;
    t.r = t.lane & 15;
    // balanced contiguous split of the fragments over the workgroups (each
    // has at least one: the grid is at most the fragment count)
    t.f_begin = (int)((int64_t)a.nfrags * blockIdx.x / gridDim.x);
    t.nf = (int)((int64_t)a.nfrags * (blockIdx.x + 1) / gridDim.x) - t.f_begin;
    t.S = t.nf * NQ;
    t.rb = BF4 ? (uint32_t)(a.K >> 1) : (uint32_t)a.K;
    t.nb = (uint32_t)(a.K >> 5);
    constexpr int SL = SROW / 4;  // scale lanes per row
    t.vo0 = (uint32_t)((t.lane ^ ((2 * t.wave) & 15)) * 16);
    t.vo1 = (uint32_t)((t.lane ^ ((2 * t.wave + 1) & 15)) * 16);
    const int sl = t.lane < 2 * SL ? t.lane : 2 * SL - 1;  // lanes past the two rows repeat the last one
    t.srow_l = 2 * t.wave + sl / SL;
    t.sbyte_l = (uint32_t)((sl % SL) * 4);

    prologue(t, std::make_integer_sequence<int, (kDecStages - 1 > NQ ? kDecStages - 1 : NQ)>{});
#pragma unroll
    for (int u = 0; u < MPW; u++) t.acc[u] = v4f{0.f, 0.f, 0.f, 0.f};

    // the first fragment (exact wait counts while A is arriving), then the rest
    fragment<true>(t, 0, std::make_integer_sequence<int, NQ>{});
    for (int f = 1; f < t.nf; f++) fragment<false>(t, f, std::make_integer_sequence<int, NQ>{});
    stage_barrier();
    if (t.wave == (t.nf - 1) % kDecWaves) reduce_store(a, smem, t.f_begin + t.nf - 1, (t.nf - 1) & 1, t.lane, t.g, t.r);
    wait_vm<0>();  // no copy into LDS may still be in flight when the workgroup ends
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
