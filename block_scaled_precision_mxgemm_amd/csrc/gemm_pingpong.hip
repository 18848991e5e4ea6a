// gemm_pingpong.hip - the large-tile GEMM for gfx950: 8 waves, 256 x 256 C
// tile, two waves per SIMD alternating between a load phase and a compute
// phase ("ping-pong").
//
// Only full tiles take this kernel (M and N multiples of 256; K a multiple of
// the slice): every copy then stays inside the operands and the copy
// addresses reduce to wave-uniform bases plus two lane offsets, which keeps
// the register budget of two waves per SIMD without spills.  (A spill would
// be fatal here: the accumulators are written by inline MFMAs whose latency
// the compiler does not know, so a spill store could read them too early.)
//
// Why: with one wave per SIMD, every stall of that wave (issuing global->LDS
// copies when the address unit is busy, waiting for LDS fragment reads, the
// barrier) idles the SIMD's matrix core; per 128-K slice the single-wave kernel
// spent ~4350 cycles in its MFMA section against 2048 of MFMA work plus ~1300
// cycles issuing copies.  Here the 8 waves form two groups of 4 (waves 0-3 and
// 4-7; waves w and w+4 share a SIMD on gfx950): while one group runs its 32
// MFMAs, the other group reads its next fragments from LDS and issues the next
// global->LDS copies, and a workgroup barrier swaps the roles.  The matrix core
// of every SIMD is fed by one of its two waves in every phase.
//
// Work split: group 0 computes C rows 0..127 of the tile, group 1 rows
// 128..255; wave s (0..3) of a group computes columns 64s..64s+63, i.e. a
// 128 x 64 sub-tile = 8 x 4 fragments of 16 x 16, 32 accumulators.
//
// LDS (two stages per region): A_top (tile rows 0..127, read by group 0 only),
// A_bot (rows 128..255, group 1 only), B (256 rows, both groups) and their
// scale rows.  Splitting A by reader lets its copies be issued three phases
// before use.  Copy schedule (phase 2s-1: group 0 loads slice s; phase 2s:
// group 1 loads slice s):
//   phase 2s-1 (issued by group 0): B(s+1)
//   phase 2s   (issued by group 1): A_top(s+2), A_bot(s+1)
// so every phase issues half a slice of copies and each region's copy has at
// least two phases between issue and first read; each group waits for its own
// copies at the end of its compute phase, before the barrier that publishes
// them.
//
// The tiled loop with double-buffered prefetch and register tiling follows
// "Treinar LLM em Swift", section "Passo 7"; data and scale planes are sliced
// together per tile as the WWDC26 session 330 summary describes (section
// "スライスと量子化行列乗算").
#include <utility>

#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

enum PPKind { kPPMX = 0, kPPF16 = 1 };

// FA_, FB_: MFMA format ids of A and B (kFmtFp8 E4M3, kFmtBf8 E5M2, kFmtFp4 E2M1).
// KSTEPS_: MFMA k-steps (128 k each) per slice; 2 only for E2M1 x E2M1, whose
// 256-k slices have the 128-byte rows (and LDS layout) of an fp8 slice.
template <int KIND, int FA_, int FB_, int KSTEPS_ = 1>
struct PPCfg {
  static constexpr int FA = FA_, FB = FB_;
  static constexpr bool AF4 = FA == kFmtFp4, BF4 = FB == kFmtFp4;
  static constexpr bool SCALED = (KIND == kPPMX);
  static constexpr bool A_FP4 = AF4, B_FP4 = BF4;
  static constexpr int KSTEPS = KSTEPS_;
  static_assert(KSTEPS == 1 || (KSTEPS == 2 && AF4 && BF4 && SCALED), "two k-steps per slice: E2M1 x E2M1 only");
  static constexpr int RA = AF4 ? 64 * KSTEPS : 128;   // bytes per A row per slice
  static constexpr int RB = BF4 ? 64 * KSTEPS : 128;
  // scale groups: 16 bytes per row, i.e. 4 / KSTEPS slices
  static constexpr int GS = 4 / KSTEPS;
  static constexpr int SZ_AH = 128 * RA;       // one A half, one stage
  static constexpr int SZ_B = 256 * RB;
  // scale buffers hold a group of 4 slices: 16 bytes per row
  static constexpr int SZ_SAH = SCALED ? 128 * 16 : 0;
  static constexpr int SZ_SB = SCALED ? 256 * 16 : 0;
  static constexpr int OFF_ATOP = 0;
  static constexpr int OFF_ABOT = OFF_ATOP + 2 * SZ_AH;
  static constexpr int OFF_B = OFF_ABOT + 2 * SZ_AH;
  static constexpr int OFF_SATOP = OFF_B + 2 * SZ_B;
  static constexpr int OFF_SABOT = OFF_SATOP + 2 * SZ_SAH;
  static constexpr int OFF_SB = OFF_SABOT + 2 * SZ_SAH;
  static constexpr int LDS_MAIN = OFF_SB + 2 * SZ_SB;
  // Epilogue staging of C (4 KiB per wave): a dedicated area when it fits,
  // else B stage 1, which is free at every tile end (see the epilogue).
  static constexpr int SZ_CST = 8 * 4096;
  static constexpr bool CST_OWN = LDS_MAIN + SZ_CST <= 160 * 1024;
  static constexpr int OFF_CST = CST_OWN ? LDS_MAIN : OFF_B + SZ_B;
  static constexpr int LDS = CST_OWN ? LDS_MAIN + SZ_CST : LDS_MAIN;
  static_assert(LDS <= 160 * 1024, "fits the 160 KiB LDS of a gfx950 CU");
  static_assert(CST_OWN || SZ_B >= SZ_CST, "C staging fits in B stage 1");
};

struct PPArgs {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  Epi e;             // output: C, bias, activation, element type
  int M, N, K;
  int tiles_m, tiles_n;
  int64_t lda, ldb;  // bytes per row
  int nslices;       // K / KSLICE (exact)
};

__device__ __forceinline__ void vm_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Barrier without a global-memory wait: the issuing group's copies stay in
// flight across it.  LDS reads of this wave complete first, so a stage read
// before the barrier may be overwritten by copies issued after it.
__device__ __forceinline__ void phase_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <class T>
struct PPKernel {
  // Lane offset of the 1 KiB tile copies.  A copy of 128-byte rows covers 8
  // rows; lane l writes LDS bytes 16l..16l+15 of it, i.e. row l/8, physical
  // chunk l%8, so it must fetch logical chunk (l%8) ^ swz8(row).  Copy q of a
  // region starts at row 8q, so swz8 = 4*(q&1) + l/16; wave sw issues copies
  // q = sw, sw+4, ..., all of parity sw&1, so one offset per wave serves all
  // its copies.  64-byte rows: 16 rows per copy, swz4 = (l/8)&3 for every q.
  template <int R>
  static __device__ __forceinline__ uint32_t lane_offset(int64_t ld, int lane, int sw) {
    if (R == 128) {
      const int c = (lane & 7) ^ ((lane >> 4) + 4 * (sw & 1));
      return (uint32_t)((lane >> 3) * ld + c * 16);
    }
    const int c = (lane & 3) ^ ((lane >> 3) & 3);
    return (uint32_t)((lane >> 2) * ld + c * 16);
  }
  // Copies of ROWS rows x R bytes of one slice, rows row0.. of the tile
  // region addressed by `rs` (a buffer resource whose base is the tile's first
  // row), split over the 4 waves of a group: wave sw issues copies sw, sw+4,
  // ...  The lane part of the address is the one loop-invariant VGPR `off`;
  // the row / slice part is a scalar offset, so no per-copy vector address
  // stays live across the K loop.
  template <int R, int ROWS>
  static __device__ __forceinline__ void copy_rows(__amdgpu_buffer_rsrc_t rs, uint32_t ld, int row0, int slice,
                                                   uint8_t* lds, int sw, uint32_t off) {
    constexpr int RPC = 1024 / R;  // rows per copy
    constexpr int NQ = ROWS / RPC;
    static_assert(NQ % 4 == 0, "copies split evenly over 4 waves");
#pragma unroll
    for (int k = 0; k < NQ / 4; k++) {
      const int q = sw + 4 * k;
      const uint32_t soff = (uint32_t)(row0 + q * RPC) * ld + (uint32_t)(slice * R);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + q * 1024), 16, off, soff, 0, 0);
    }
  }
  // Scale bytes of a group of 4 slices: 16 per row (4 blocks per slice), 64
  // rows per copy from row `row` of the tile, into lds (wave-uniform).  A
  // copy of one slice's 4 bytes per row would touch one cache line per row
  // for 256 bytes; taking 4 slices at once quarters the line requests (the
  // per-slice scale copies cost about 14 % of a large GEMM's time,
  // measured).  Past the end of K the 16 bytes run into the next row, or past
  // the last row into the buffer's end (read as zeros); they are not used.
  static __device__ __forceinline__ void copy_scale_group(__amdgpu_buffer_rsrc_t rs, uint32_t nb, int row, int G,
                                                          uint8_t* lds, uint32_t off) {
    const uint32_t soff = (uint32_t)row * nb + (uint32_t)(G * 16);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, off, soff, 0, 0);
  }

  template <int R>
  static __device__ __forceinline__ v8i read_frag(const uint8_t* lds, int row, int g) {
    v8i f;
    if (R == 128) {
      const int s = swz8(row);
      const v4i lo = *reinterpret_cast<const v4i*>(lds + row * 128 + ((g ^ s) << 4));
      const v4i hi = *reinterpret_cast<const v4i*>(lds + row * 128 + (((4 + g) ^ s) << 4));
      f = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      const v4i lo = *reinterpret_cast<const v4i*>(lds + row * 64 + ((g ^ swz4(row)) << 4));
      f = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
    }
    return f;
  }

  // The 32 scaled MFMAs of one slice, B fragment j outer; the scale byte
  // index must be an immediate, hence the index sequence.
  template <int... I>
  static __device__ __forceinline__ void compute_scaled(v4f (&acc)[8][4], const v8i (&af)[8], const v8i (&bf)[4],
                                                        const int (&sa)[2], int sb, std::integer_sequence<int, I...>) {
    constexpr int FB = T::FB, FA = T::FA;
    (mfma_scaled_acc_pk<FB, FA, I / 8, (I % 8) & 3>(acc[I % 8][I / 8], bf[I / 8], af[I % 8], sb, sa[(I % 8) >> 2]),
     ...);
  }
  // E2M1 operand of k-step H of a 128-byte fragment row: bytes 16 lg .. of
  // the step's 64 (H = 0: the fragment's first half, H = 1: its second)
  template <int H>
  static __device__ __forceinline__ v8i fp4_step(const v8i& f) {
    return v8i{f[4 * H], f[4 * H + 1], f[4 * H + 2], f[4 * H + 3], 0, 0, 0, 0};
  }
  template <int H, int... I>
  static __device__ __forceinline__ void compute_scaled_step(v4f (&acc)[8][4], const v8i (&af)[8], const v8i (&bf)[4],
                                                             const int (&sa)[2], int sb,
                                                             std::integer_sequence<int, I...>) {
    constexpr int FB = T::FB, FA = T::FA;
    (mfma_scaled_acc_pk<FB, FA, I / 8, (I % 8) & 3>(acc[I % 8][I / 8], fp4_step<H>(bf[I / 8]), fp4_step<H>(af[I % 8]),
                                                    sb, sa[(I % 8) >> 2]),
     ...);
  }

  static __device__ __forceinline__ void run(const PPArgs& a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform role: scalar registers and scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, sw = wave & 3;
    const int lg = lane >> 4, r = lane & 15;
    const int S = a.nslices;
    const int nb = a.K >> 5;
    const int total = a.tiles_m * a.tiles_n;

    const uint32_t oa = lane_offset<T::RA>(a.lda, lane, sw);
    const uint32_t ob = lane_offset<T::RB>(a.ldb, lane, sw);
    const uint32_t os = (uint32_t)(lane * nb);
    // Buffer resources over the current tile's 256 rows of A, B and their
    // scales (word 3: the raw-buffer format of gfx9-class resources).
    constexpr int kRsrcWord3 = 0x00020000;
    const uint32_t lda = (uint32_t)a.lda, ldb = (uint32_t)a.ldb;
    int m0 = 0, n0 = 0;
    __amdgpu_buffer_rsrc_t rs_a, rs_b, rs_sa, rs_sb;
    auto set_tile = [&](int tile) {
      int tm, tn;
      tile_of_block(tile, a.tiles_m, a.tiles_n, tm, tn);
      m0 = tm * 256;
      n0 = tn * 256;
      rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)(a.A + (int64_t)m0 * lda), 0, 256 * lda, kRsrcWord3);
      rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)(a.B + (int64_t)n0 * ldb), 0, 256 * ldb, kRsrcWord3);
      if (T::SCALED) {
        rs_sa = __builtin_amdgcn_make_buffer_rsrc((void*)(a.SA + (int64_t)m0 * nb), 0, 256 * nb, kRsrcWord3);
        rs_sb = __builtin_amdgcn_make_buffer_rsrc((void*)(a.SB + (int64_t)n0 * nb), 0, 256 * nb, kRsrcWord3);
      }
    };
    // copies of slice t of each region (issued by the 4 waves of the calling group)
    auto copy_atop = [&](int t) {
      copy_rows<T::RA, 128>(rs_a, lda, 0, t, smem + T::OFF_ATOP + (t & 1) * T::SZ_AH, sw, oa);
    };
    auto copy_abot = [&](int t) {
      copy_rows<T::RA, 128>(rs_a, lda, 128, t, smem + T::OFF_ABOT + (t & 1) * T::SZ_AH, sw, oa);
    };
    auto copy_b = [&](int t) {
      copy_rows<T::RB, 256>(rs_b, ldb, 0, t, smem + T::OFF_B + (t & 1) * T::SZ_B, sw, ob);
    };
    // Scale group G (slices 4G .. 4G + 3) into buffer G & 1 of each region,
    // one copy of 64 rows per wave of the calling group: A_top rows 0-127
    // (waves 0, 1) and A_bot rows 128-255 (waves 2, 3), or B rows 64 sw...
    // Group G + 1 is copied in the load phase of slice 4G + 1 (A by group 1,
    // B by group 0), after the last reads of group G - 1 from that buffer
    // (slice 4G - 1) and well before its first reads (slice 4G + 4).
    auto copy_sa_group = [&](int G) {
      const int half = sw >> 1, q = sw & 1;
      copy_scale_group(rs_sa, nb, half * 128 + q * 64, G,
                       smem + (half ? T::OFF_SABOT : T::OFF_SATOP) + (G & 1) * T::SZ_SAH + q * 1024, os);
    };
    auto copy_sb_group = [&](int G) {
      copy_scale_group(rs_sb, nb, sw * 64, G, smem + T::OFF_SB + (G & 1) * T::SZ_SB + sw * 1024, os);
    };
    const int ng = T::KSTEPS == 1 ? (S + 3) >> 2 : (S + 1) >> 1;  // scale groups

    // The workgroup is persistent: it takes tiles blockIdx.x, + gridDim.x, ...
    // (the grid is at most one workgroup per CU), so there is no dispatch gap
    // between tiles, and the copies that start a tile are issued by group 0
    // while group 1 still runs the previous tile's last compute phase.
    int tile = blockIdx.x;
    set_tile(tile);
    // prologue of the first tile: the slices needed before the copies of the
    // steady state (B(0), A_top(0), A_top(1), A_bot(0)), issued by both groups
    if (grp == 0) {
      copy_b(0);
      if (T::SCALED) copy_sb_group(0);
    } else {
      copy_atop(0);
      if (S > 1) copy_atop(1);
      copy_abot(0);
      if (T::SCALED) copy_sa_group(0);
    }
    vm_wait_all();
    phase_barrier();

    v4f acc[8][4];
    for (;;) {
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    mfma_fence_init(acc);

    // Each wave runs: load slice s (LDS -> registers, issue its share of the
    // next copies), barrier, compute slice s, barrier.  Group 1 starts one
    // phase late (an extra barrier first, none after its last compute), so at
    // every phase one group loads while the other computes.  Both groups pass
    // 2S barriers.
    if (grp == 1) phase_barrier();
    for (int s = 0; s < S; s++) {
      const int st = s & 1;
      v8i af[8], bf[4];
      // scale bytes packed four to a register: byte i&3 of sa[i>>2] belongs
      // to A fragment i, byte j of sb to B fragment j (k-step 1 of a two-step
      // slice: sa1, sb1)
      int sa[2] = {0, 0}, sb = 0;
      int sa1[2] = {0, 0}, sb1 = 0;
      {
        const uint8_t* la = smem + (grp ? T::OFF_ABOT : T::OFF_ATOP) + st * T::SZ_AH;
        const uint8_t* lb = smem + T::OFF_B + st * T::SZ_B;
#pragma unroll
        for (int i = 0; i < 8; i++) af[i] = read_frag<T::RA>(la, i * 16 + r, lg);
#pragma unroll
        for (int j = 0; j < 4; j++) bf[j] = read_frag<T::RB>(lb, sw * 64 + j * 16 + r, lg);
        if (T::SCALED && T::KSTEPS == 1) {
          // slice s: group buffer (s >> 2) & 1, bytes 4 (s & 3) + lg of each row
          const int sg = (s >> 2) & 1, sk = (s & 3) * 4 + lg;
          const uint8_t* lsa = smem + (grp ? T::OFF_SABOT : T::OFF_SATOP) + sg * T::SZ_SAH;
          const uint8_t* lsb = smem + T::OFF_SB + sg * T::SZ_SB;
          uint32_t x[8], y[4];
#pragma unroll
          for (int i = 0; i < 8; i++) x[i] = lsa[(i * 16 + r) * 16 + sk];
#pragma unroll
          for (int j = 0; j < 4; j++) y[j] = lsb[(sw * 64 + j * 16 + r) * 16 + sk];
          sa[0] = (int)(x[0] | (x[1] << 8) | (x[2] << 16) | (x[3] << 24));
          sa[1] = (int)(x[4] | (x[5] << 8) | (x[6] << 16) | (x[7] << 24));
          sb = (int)(y[0] | (y[1] << 8) | (y[2] << 16) | (y[3] << 24));
        } else if (T::SCALED) {
          // two k-steps: group buffer (s >> 1) & 1, bytes 8 (s & 1) + 4 h + lg
          // of each row for step h;
          const int sg = (s >> 1) & 1, sk = (s & 1) * 8 + lg;
          const uint8_t* lsa = smem + (grp ? T::OFF_SABOT : T::OFF_SATOP) + sg * T::SZ_SAH;
          const uint8_t* lsb = smem + T::OFF_SB + sg * T::SZ_SB;
          // step 0 here; step 1 after this phase's copies (below), so that the
          // two steps' byte temporaries are never live together
          uint32_t x[8], y[4];
#pragma unroll
          for (int i = 0; i < 8; i++) x[i] = lsa[(i * 16 + r) * 16 + sk];
#pragma unroll
          for (int j = 0; j < 4; j++) y[j] = lsb[(sw * 64 + j * 16 + r) * 16 + sk];
          sa[0] = (int)(x[0] | (x[1] << 8) | (x[2] << 16) | (x[3] << 24));
          sa[1] = (int)(x[4] | (x[5] << 8) | (x[6] << 16) | (x[7] << 24));
          sb = (int)(y[0] | (y[1] << 8) | (y[2] << 16) | (y[3] << 24));
        }
        if (grp == 0) {
          if (s + 1 < S) copy_b(s + 1);
        } else {
          if (s + 2 < S) copy_atop(s + 2);
          if (s + 1 < S) copy_abot(s + 1);
        }
        if constexpr (T::KSTEPS == 1) {
          if (T::SCALED && (s & 3) == 1 && (s >> 2) + 1 < ng) {
            if (grp == 0)
              copy_sb_group((s >> 2) + 1);
            else
              copy_sa_group((s >> 2) + 1);
          }
        } else if ((s & 1) == 0 && (s >> 1) + 1 < ng) {
          // groups of 2 slices: group G + 1 in slice 2G, after the last reads
          // of group G - 1 (slice 2G - 1) and two slices before its first
          // reads (slice 2G + 2)
          if (grp == 0)
            copy_sb_group((s >> 1) + 1);
          else
            copy_sa_group((s >> 1) + 1);
        }
        if constexpr (T::SCALED && T::KSTEPS == 2) {
          // the step-1 scale bytes: after the copies are issued and the step-0
          // bytes are packed (the fence keeps the loads below it)
          asm volatile("" : "+v"(sa[0]), "+v"(sa[1]), "+v"(sb)::"memory");
          const int sg = (s >> 1) & 1, sk = (s & 1) * 8 + 4 + lg;
          const uint8_t* lsa = smem + (grp ? T::OFF_SABOT : T::OFF_SATOP) + sg * T::SZ_SAH;
          const uint8_t* lsb = smem + T::OFF_SB + sg * T::SZ_SB;
          uint32_t x[8], y[4];
#pragma unroll
          for (int i = 0; i < 8; i++) x[i] = lsa[(i * 16 + r) * 16 + sk];
#pragma unroll
          for (int j = 0; j < 4; j++) y[j] = lsb[(sw * 64 + j * 16 + r) * 16 + sk];
          sa1[0] = (int)(x[0] | (x[1] << 8) | (x[2] << 16) | (x[3] << 24));
          sa1[1] = (int)(x[4] | (x[5] << 8) | (x[6] << 16) | (x[7] << 24));
          sb1 = (int)(y[0] | (y[1] << 8) | (y[2] << 16) | (y[3] << 24));
        }
      }
      if constexpr (T::SCALED && T::KSTEPS == 2) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_nop 4"
                     : "+v"(sa[0]), "+v"(sa[1]), "+v"(sb), "+v"(sa1[0]), "+v"(sa1[1]), "+v"(sb1)::"memory");
      } else if constexpr (T::SCALED) {
        // The barrier asm takes the packed scales as operands, so the packing
        // (VALU) stays in the load phase instead of being sunk into the
        // compute phase; the s_nop keeps the wait states an MFMA needs after
        // a VALU write of its operand, which the compiler does not insert for
        // inline MFMAs.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_nop 4" : "+v"(sa[0]), "+v"(sa[1]), "+v"(sb)::"memory");
      } else {
        phase_barrier();
      }
      if constexpr (T::SCALED && T::KSTEPS == 2) {
        compute_scaled_step<0>(acc, af, bf, sa, sb, std::make_integer_sequence<int, 32>{});
        compute_scaled_step<1>(acc, af, bf, sa1, sb1, std::make_integer_sequence<int, 32>{});
      } else if constexpr (T::SCALED) {
        compute_scaled(acc, af, bf, sa, sb, std::make_integer_sequence<int, 32>{});
      } else {
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
          for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < 8; i++) {
              const v4i bq = h ? v4i{bf[j][4], bf[j][5], bf[j][6], bf[j][7]} : v4i{bf[j][0], bf[j][1], bf[j][2], bf[j][3]};
              const v4i aq = h ? v4i{af[i][4], af[i][5], af[i][6], af[i][7]} : v4i{af[i][0], af[i][1], af[i][2], af[i][3]};
              mfma_f16_acc_v(acc[i][j], bq, aq);
            }
      }
      vm_wait_all();  // this group's copies issued in this slice's load phase
      if (grp == 0 || s + 1 < S) phase_barrier();
    }
    mfma_drain(acc);

    // ---- epilogue (full tiles only) -----------------------------------------
    // Lane (lg, r) holds C[m][n .. n+3] of fragment (i, j): row m = i*16 + r
    // of this wave's 128 rows, columns n = j*16 + 4*lg of its 64.  Stored as
    // is, every store instruction would write 64 bytes to each of 16 rows,
    // half cache lines, when all CUs write their tiles at the same moment.
    // Each 16 x 64 block (one i) therefore goes through this wave's 4 KiB of
    // LDS (16-byte chunks XOR-swizzled by row: conflict-free both ways) and
    // comes back row-contiguous: each store writes 256 bytes to each of 4
    // rows.  The staging area is either unused by the tile loop or B stage 1:
    // every read of the finished tile's B stages has completed (group 1's last
    // load phase ended with a barrier before either group gets here), the next
    // tile's first copies go to B stage 0 and the A regions, and its first
    // copy into B stage 1 is issued after the barrier that ends this epilogue.
    {
      uint8_t* cst = smem + T::OFF_CST + wave * 4096;
      // the epilogue's lane-dependent addresses are derived here, from a lane
      // index the compiler cannot see through, so they are not hoisted out of
      // the tile loop and kept live (in registers the K loop needs)
      int le = lane;
      if constexpr (T::KSTEPS == 2) {
        // recomputed rather than kept: holding the lane index across the
        // two-step K loop would spill it
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(le));
      } else {
        asm volatile("" : "+v"(le));
      }
      const int lr = le & 15, llg = le >> 4;     // the fragment layout's (r, lg)
      const int rr = le >> 4, cc = le & 15;      // read-back: row-in-quad, 16-byte chunk
      // every store of this lane covers columns nc .. nc+3: its bias is
      // loaded once per tile
      const int nc = n0 + sw * 64 + cc * 4;
      const bool plain = epi_plain(a.e);
      v4f bias4 = {0.f, 0.f, 0.f, 0.f};
      if (a.e.bias != nullptr) bias4 = *reinterpret_cast<const v4f*>(a.e.bias + nc);
#pragma unroll
      for (int i = 0; i < 8; i++) {
#pragma unroll
        for (int j = 0; j < 4; j++)
          *reinterpret_cast<v4f*>(cst + lr * 256 + (((j * 4 + llg) ^ lr) << 4)) = acc[i][j];
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int row = q * 4 + rr;
          v4f v = *reinterpret_cast<const v4f*>(cst + row * 256 + ((cc ^ row) << 4));
          const int64_t m = m0 + grp * 128 + i * 16 + row;
          // non-temporal: C is not read again here, and all CUs write their
          // tiles at once; keeping it out of the normal cache retention
          // leaves L2 to the A and B tiles (4.7 % faster at 8192^3, 6.7 % on
          // 8192 x 14336 x 4096, measured)
          if (plain) {
            __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(reinterpret_cast<float*>(a.e.C) + m * a.N + nc));
          } else {
            v += bias4;
            if (a.e.act == kActGelu) {
#pragma unroll
              for (int t = 0; t < 4; t++) v[t] = gelu(v[t]);
            }
            epi_put4<true>(a.e, a.N, m, nc, v, true);
          }
        }
      }
    }
    const int next = tile + (int)gridDim.x;
    if (next >= total) break;
    tile = next;
    set_tile(tile);
    // Group 0 finished its part of the tile one phase before group 1; every
    // LDS read of the finished tile and every copy into LDS has completed
    // (each group waited for its copies and passed the barrier after group
    // 1's last load phase), so group 0 issues the next tile's prologue copies
    // now, over group 1's last compute phase.  Its wait also covers its C
    // stores; group 1's C stores are covered by its first wait of the next
    // tile.
    if (grp == 0) {
      copy_b(0);
      copy_atop(0);
      if (S > 1) copy_atop(1);
      copy_abot(0);
      if (T::SCALED) {
        copy_sb_group(0);
        copy_sa_group(0);
      }
      vm_wait_all();
    }
    phase_barrier();
    }
  }
};

template <class T>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void pingpong_kernel(PPArgs a) {
  PPKernel<T>::run(a);
}

// ---- 128 x 128 tiles, K split between the groups --------------------------
//
// Outputs with too few 256 x 256 tiles for the chip (2048^3 has 64) take one
// workgroup per 128 x 128 tile with the same 8-wave ping-pong, but both groups
// compute the whole tile: group 0 the even K slices, group 1 the odd ones,
// each wave a 64 x 64 sub-tile (4 x 4 fragments, 64 accumulator registers).
// Each group double-buffers its own slices (A, B and scale rows of one slice
// per stage), so while one group reads fragments and issues its next copies
// the other runs its 16 MFMAs, as in the 256 x 256 kernel; a single-group
// 128 x 128 kernel instead spends its copy issue, fragment reads and MFMAs in
// series.  At the end group 1 passes its partial sums to group 0 through LDS
// and group 0 adds them (its own first, a fixed order) and stores the tile
// through the epilogue.
template <class T>
struct PP128Kernel {
  using P = PPKernel<T>;
  static constexpr int SZ_A = 128 * T::RA, SZ_B = 128 * T::RB;
  static constexpr int SZ_STAGE = SZ_A + SZ_B;
  // one scale buffer: a group of 4 slices, 16 bytes per row, A then B
  static constexpr int SZ_SG = T::SCALED ? 2 * 128 * 16 : 0;
  static constexpr int SZ_GROUP = 2 * SZ_STAGE + 2 * SZ_SG;
  static constexpr int SZ_RED = 4 * 16 * 64 * 16;  // group 1's partials: 4 waves x 16 fragments x 64 lanes
  static constexpr int SZ_CST = 8 * 4096;  // epilogue staging, 4 KiB per wave, after the partials
  static constexpr int LDS = 2 * SZ_GROUP > SZ_RED + SZ_CST ? 2 * SZ_GROUP : SZ_RED + SZ_CST;
  static_assert(LDS <= 160 * 1024, "fits the 160 KiB LDS of a gfx950 CU");

  template <int... I>
  static __device__ __forceinline__ void compute_scaled(v4f (&acc)[4][4], const v8i (&af)[4], const v8i (&bf)[4],
                                                        int sa, int sb, std::integer_sequence<int, I...>) {
    (mfma_scaled_acc_pk<T::FB, T::FA, I / 4, I % 4>(acc[I % 4][I / 4], bf[I / 4], af[I % 4], sb, sa), ...);
  }

  static __device__ __forceinline__ void run(const PPArgs& a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2, sw = wave & 3;
    const int lg = lane >> 4, r = lane & 15;
    const int S = a.nslices;
    const int S0 = (S + 1) / 2;              // group 0 takes slices 0, 2, ...
    const int Sg = grp == 0 ? S0 : S / 2;    // group 1 takes slices 1, 3, ...
    const int nb = a.K >> 5;
    int tm, tn;
    tile_of_block(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * 128, n0 = tn * 128;

    constexpr int kRsrcWord3 = 0x00020000;
    const uint32_t lda = (uint32_t)a.lda, ldb = (uint32_t)a.ldb;
    const auto rs_a = __builtin_amdgcn_make_buffer_rsrc((void*)(a.A + (int64_t)m0 * lda), 0, 128 * lda, kRsrcWord3);
    const auto rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)(a.B + (int64_t)n0 * ldb), 0, 128 * ldb, kRsrcWord3);
    __amdgpu_buffer_rsrc_t rs_sa = rs_a, rs_sb = rs_b;
    if (T::SCALED) {
      rs_sa = __builtin_amdgcn_make_buffer_rsrc((void*)(a.SA + (int64_t)m0 * nb), 0, 128 * nb, kRsrcWord3);
      rs_sb = __builtin_amdgcn_make_buffer_rsrc((void*)(a.SB + (int64_t)n0 * nb), 0, 128 * nb, kRsrcWord3);
    }
    const uint32_t oa = P::template lane_offset<T::RA>(a.lda, lane, sw);
    // equal row sizes come with equal strides in every launch
    const uint32_t ob = (T::RA == T::RB) ? oa : P::template lane_offset<T::RB>(a.ldb, lane, sw);
    const uint32_t os = (uint32_t)(lane * nb);
    uint8_t* gbase = smem + grp * SZ_GROUP;

    // copies of this group's iteration i (slice 2i + grp) into its stage i & 1
    auto copy_iter = [&](int i) {
      const int k = 2 * i + grp;
      uint8_t* st = gbase + (i & 1) * SZ_STAGE;
      P::template copy_rows<T::RA, 128>(rs_a, lda, 0, k, st, sw, oa);
      P::template copy_rows<T::RB, 128>(rs_b, ldb, 0, k, st + SZ_A, sw, ob);
    };
    // Scale group G (slices 4G .. 4G + 3, this group's iterations 2G and
    // 2G + 1) into the group's buffer G & 1: one copy of 64 rows x 16 bytes
    // per wave (A rows for waves 0, 1, B rows for waves 2, 3).  Group G + 1
    // is copied in iteration 2G, after the last use of the buffer (group
    // G - 1, iteration 2G - 1) and two iterations before its first use.
    auto copy_sgroup = [&](int G) {
      const int op = sw >> 1, q = sw & 1;
      P::copy_scale_group(op ? rs_sb : rs_sa, nb, q * 64, G,
                          gbase + 2 * SZ_STAGE + (G & 1) * SZ_SG + op * 2048 + q * 1024, os);
    };
    if (Sg > 0) {
      copy_iter(0);
      if (T::SCALED) copy_sgroup(0);
    }
    vm_wait_all();
    phase_barrier();

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    mfma_fence_init(acc);

    // Barrier pairing: group 0's load phase of iteration i meets group 1's
    // compute phase of iteration i - 1 and the other way round; group 1
    // starts one phase late and skips the barrier after its last compute,
    // then both groups pad to the 2 S0 barriers of group 0's loop.
    int nbar = 0;
    if (grp == 1) {
      phase_barrier();
      nbar = 1;
    }
    const int wr = (sw >> 1) * 64, wc = (sw & 1) * 64;  // this wave's sub-tile
    for (int i = 0; i < Sg; i++) {
      const uint8_t* st = gbase + (i & 1) * SZ_STAGE;
      v8i af[4], bf[4];
      int sa = 0, sb = 0;
#pragma unroll
      for (int f = 0; f < 4; f++) af[f] = P::template read_frag<T::RA>(st, wr + 16 * f + r, lg);
#pragma unroll
      for (int f = 0; f < 4; f++) bf[f] = P::template read_frag<T::RB>(st + SZ_A, wc + 16 * f + r, lg);
      if (T::SCALED) {
        // slice 2i + grp: buffer (i >> 1) & 1, bytes 4 ((2i + grp) & 3) + lg of each row
        const uint8_t* lsa = gbase + 2 * SZ_STAGE + ((i >> 1) & 1) * SZ_SG;
        const uint8_t* lsb = lsa + 2048;
        const int sk = (2 * (i & 1) + grp) * 4 + lg;
        uint32_t x[4], y[4];
#pragma unroll
        for (int f = 0; f < 4; f++) x[f] = lsa[(wr + 16 * f + r) * 16 + sk];
#pragma unroll
        for (int f = 0; f < 4; f++) y[f] = lsb[(wc + 16 * f + r) * 16 + sk];
        sa = (int)(x[0] | (x[1] << 8) | (x[2] << 16) | (x[3] << 24));
        sb = (int)(y[0] | (y[1] << 8) | (y[2] << 16) | (y[3] << 24));
      }
      if (i + 1 < Sg) copy_iter(i + 1);
      if (T::SCALED && (i & 1) == 0 && i + 2 < Sg) copy_sgroup((i >> 1) + 1);
      if constexpr (T::SCALED) {
        // as in the 256 x 256 kernel: the packed scales are operands of the
        // barrier, and s_nop covers the VALU-write -> MFMA-read wait states
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_nop 4" : "+v"(sa), "+v"(sb)::"memory");
      } else {
        phase_barrier();
      }
      nbar++;
      if constexpr (T::SCALED) {
        compute_scaled(acc, af, bf, sa, sb, std::make_integer_sequence<int, 16>{});
      } else {
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
          for (int j = 0; j < 4; j++)
#pragma unroll
            for (int f = 0; f < 4; f++) {
              const v4i bq = h ? v4i{bf[j][4], bf[j][5], bf[j][6], bf[j][7]} : v4i{bf[j][0], bf[j][1], bf[j][2], bf[j][3]};
              const v4i aq = h ? v4i{af[f][4], af[f][5], af[f][6], af[f][7]} : v4i{af[f][0], af[f][1], af[f][2], af[f][3]};
              mfma_f16_acc_v(acc[f][j], bq, aq);
            }
      }
      vm_wait_all();  // this group's copies for iteration i + 1
      if (grp == 0 || i + 1 < Sg) {
        phase_barrier();
        nbar++;
      }
    }
    for (; nbar < 2 * S0; nbar++) phase_barrier();
    mfma_drain(acc);

    // every load phase and copy has completed: the stages are free.  The
    // groups split the store: group 0 finishes row blocks i = 0, 1 of its
    // sub-tile and group 1 blocks 2, 3, each after adding the other group's
    // partial sums of those blocks, passed through LDS (8 KiB per wave); the
    // sum is group 0's plus group 1's either way.
    const int ikeep = 2 * grp;
    v4f* give = reinterpret_cast<v4f*>(smem) + (grp * 4 + sw) * 8 * 64 + lane;
    const v4f* take = reinterpret_cast<const v4f*>(smem) + ((1 - grp) * 4 + sw) * 8 * 64 + lane;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) give[(i * 4 + j) * 64] = grp ? acc[i][j] : acc[2 + i][j];
    phase_barrier();
    // Lane (lg, r) of fragment (i, j) holds C[m][n .. n+3] with m = 16 i + r
    // of the sub-tile's rows and n = 16 j + 4 lg of its columns.  Each 16 x
    // 64 block (one i) goes through 4 KiB of this wave's LDS (16-byte chunks
    // XOR-swizzled by row) and comes back row-contiguous, so that every store
    // writes 256 bytes to each of 4 rows (whole cache lines) instead of 64
    // bytes to each of 16.
    uint8_t* cst = smem + SZ_RED + wave * 4096;
    int le = lane;
    asm volatile("" : "+v"(le));
    const int lr = le & 15, llg = le >> 4;  // the fragment layout's (r, lg)
    const int rr = le >> 4, cc = le & 15;   // read-back: row-in-quad, 16-byte chunk
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int i = ikeep + h;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const v4f mine = grp ? acc[2 + h][j] : acc[h][j];
        const v4f other = take[(h * 4 + j) * 64];
        *reinterpret_cast<v4f*>(cst + lr * 256 + (((j * 4 + llg) ^ lr) << 4)) = grp ? other + mine : mine + other;
      }
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int row = q * 4 + rr;
        const v4f v = *reinterpret_cast<const v4f*>(cst + row * 256 + ((cc ^ row) << 4));
        epi_store4<true>(a.e, a.N, m0 + wr + 16 * i + row, n0 + wc + 4 * cc, v, true);
      }
    }
  }
};

template <class T>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void pp128_kernel(PPArgs a) {
  PP128Kernel<T>::run(a);
}

template <class T>
hipError_t launch_pp128(PPArgs a, int kslice, hipStream_t stream) {
  a.tiles_m = a.M / 128;
  a.tiles_n = a.N / 128;
  a.nslices = a.K / kslice;
  const int tiles = a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((pp128_kernel<T>), dim3((unsigned)tiles), dim3(512), 0, stream, a);
  return hipGetLastError();
}

template <class T>
hipError_t launch_pp(PPArgs a, int kslice, hipStream_t stream) {
  a.tiles_m = (a.M + 255) / 256;
  a.tiles_n = (a.N + 255) / 256;
  a.nslices = a.K / kslice;
  // one persistent workgroup per CU (the LDS use allows one), at most one per tile
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int tiles = a.tiles_m * a.tiles_n;
  const int grid = (cus > 0 && cus < tiles) ? cus : tiles;
  hipLaunchKernelGGL((pingpong_kernel<T>), dim3((unsigned)grid), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

bool pingpong_mx_ok(const uint8_t* SA, const uint8_t* SB, int64_t M, int64_t N, int64_t K) {
  return (M % 256) == 0 && (N % 256) == 0 && (K % 128) == 0 && (((uintptr_t)SA | (uintptr_t)SB) & 3) == 0;
}

bool pp128_mx_ok(const uint8_t* SA, const uint8_t* SB, int64_t M, int64_t N, int64_t K) {
  return (M % 128) == 0 && (N % 128) == 0 && (K % 128) == 0 && (((uintptr_t)SA | (uintptr_t)SB) & 3) == 0;
}

hipError_t launch_mx_pingpong(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                              int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream) {
  PPArgs a{};
  a.A = (const uint8_t*)A;
  a.SA = SA;
  a.B = (const uint8_t*)B;
  a.SB = SB;
  a.e = e;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.lda = (fmt == 2) ? K / 2 : K;
  a.ldb = (fmt == 1 || fmt == 2) ? K / 2 : K;
  switch (fmt) {
    case 0: return launch_pp<PPCfg<kPPMX, kFmtFp8, kFmtFp8>>(a, 128, stream);
    case 1: return launch_pp<PPCfg<kPPMX, kFmtFp8, kFmtFp4>>(a, 128, stream);
    case 2:
      // 256-k slices (two MFMA k-steps per phase) where K allows
      return (K % 256) == 0 ? launch_pp<PPCfg<kPPMX, kFmtFp4, kFmtFp4, 2>>(a, 256, stream)
                            : launch_pp<PPCfg<kPPMX, kFmtFp4, kFmtFp4>>(a, 128, stream);
    case 3: return launch_pp<PPCfg<kPPMX, kFmtBf8, kFmtBf8>>(a, 128, stream);
    case 4: return launch_pp<PPCfg<kPPMX, kFmtFp8, kFmtBf8>>(a, 128, stream);
    default: return launch_pp<PPCfg<kPPMX, kFmtBf8, kFmtFp8>>(a, 128, stream);
  }
}

hipError_t launch_mx_pp128(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                           int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream) {
  PPArgs a{};
  a.A = (const uint8_t*)A;
  a.SA = SA;
  a.B = (const uint8_t*)B;
  a.SB = SB;
  a.e = e;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.lda = (fmt == 2) ? K / 2 : K;
  a.ldb = (fmt == 1 || fmt == 2) ? K / 2 : K;
  switch (fmt) {
    case 0: return launch_pp128<PPCfg<kPPMX, kFmtFp8, kFmtFp8>>(a, 128, stream);
    case 1: return launch_pp128<PPCfg<kPPMX, kFmtFp8, kFmtFp4>>(a, 128, stream);
    case 2: return launch_pp128<PPCfg<kPPMX, kFmtFp4, kFmtFp4>>(a, 128, stream);
    case 3: return launch_pp128<PPCfg<kPPMX, kFmtBf8, kFmtBf8>>(a, 128, stream);
    case 4: return launch_pp128<PPCfg<kPPMX, kFmtFp8, kFmtBf8>>(a, 128, stream);
    default: return launch_pp128<PPCfg<kPPMX, kFmtBf8, kFmtFp8>>(a, 128, stream);
  }
}

hipError_t launch_f16_pp128(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N, int64_t K,
                            hipStream_t stream) {
  PPArgs a{};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.e = Epi{C, nullptr, kOutF32, kActNone};
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.lda = K * 2;
  a.ldb = K * 2;
  return launch_pp128<PPCfg<kPPF16, kFmtFp8, kFmtFp8>>(a, 64, stream);
}

hipError_t launch_f16_pingpong(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N, int64_t K,
                               hipStream_t stream) {
  PPArgs a{};
  a.A = (const uint8_t*)A;
  a.B = (const uint8_t*)B;
  a.e = Epi{C, nullptr, kOutF32, kActNone};
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.lda = K * 2;
  a.ldb = K * 2;
  return launch_pp<PPCfg<kPPF16, kFmtFp8, kFmtFp8>>(a, 64, stream);
}

}  // namespace mxg
