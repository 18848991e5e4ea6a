// gemm_tiled.hip - LDS-tiled GEMM kernels for large M: the scaled-MFMA MX
// GEMM (the product path), the dense fp16 comparison GEMM and the
// dequantize-to-fp16 ablation.  All three share one skeleton:
//
//   * a workgroup of 4 waves owns a BM x BN tile of C; each wave owns a
//     (BM/WM) x (BN/WN) sub-tile held in MFMA accumulators;
//   * the K loop walks slices of 128 K elements (MX operands: 128 bytes of
//     fp8 codes or 64 bytes of packed fp4 per row) or of 64 K elements (fp16:
//     128 bytes per row) through two LDS stages: the copy of slice s+1 (direct
//     global->LDS 16-byte loads, no register staging) overlaps the MFMAs on
//     slice s; one barrier per slice;
//   * LDS rows are 16-byte-chunk XOR-swizzled so that both the tile copies and
//     the fragment reads are bank-conflict free;
//   * the scale planes (4 UE8M0 bytes per row per slice) travel through
//     registers into LDS next to their data, sliced together with it as the
//     WWDC26 session 330 summary describes for multi-plane tensors (section
//     "スライスと量子化行列乗算");
//   * the MFMA's first source is the B fragment, so each lane's 4 accumulator
//     values are 4 consecutive columns of one C row: the epilogue stores
//     16-byte vectors.
//
// The tiled loop with zero-padded edge tiles and a barrier per tile follows
// "Treinar LLM em Swift", sections "Passo 4" (threadgroup tiling) and
// "Passo 7" (register tiling and double-buffered prefetch), re-designed for
// 64-wide waves, 160 KiB of LDS and the CDNA4 MFMA units.
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

enum Kind { kMX = 0, kF16 = 1, kDEQ = 2 };

// FA_, FB_: MFMA format ids of the MX operands (kFmtFp8 E4M3, kFmtBf8 E5M2,
// kFmtFp4 E2M1); unused by the fp16 kinds
template <int KIND, int BM_, int BN_, int WM_, int WN_, int FA_, int FB_, bool BKN_>
struct Cfg {
  static constexpr int KIND_ = KIND;
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int FA = FA_, FB = FB_;
  static constexpr bool AF4 = FA == kFmtFp4, BF4 = FB == kFmtFp4, BKN = BKN_;
  // FP6 (E2M3 / E3M2) right operand: 96 bytes per row and 128-k slice,
  // copied 12 bytes per lane into the 16-byte slots of 128-byte LDS rows
  static constexpr bool B6 = FB == kFmtFp6 || FB == kFmtBf6;
  // INT4 right operand: 64 bytes per row and slice (as E2M1), remapped in
  // registers to the E4M3 codes of the same values for an E4M3 MFMA operand
  static constexpr bool BI4 = FB == kElemInt4;
  // INT2 right operand: 32 bytes per row and slice, remapped to E2M1 codes
  static constexpr bool BI2 = FB == kElemInt2;
  static constexpr int FBM = BI4 ? kFmtFp8 : BI2 ? kFmtFp4 : FB;  // MFMA format of the right operand
  static constexpr bool SCALED = (KIND != kF16);
  static constexpr int TM = BM / WM, TN = BN / WN;   // wave sub-tile
  static constexpr int FM = TM / 16, FN = TN / 16;   // 16x16 fragments per wave
  static constexpr int RA = AF4 ? 64 : 128;          // LDS bytes per A row per slice
  static constexpr int RB = BI2 ? 32 : (BF4 || BI4) ? 64 : 128;
  static constexpr int KSLICE = (KIND == kF16) ? 64 : 128;  // K elements per slice
  static constexpr int SZA = BM * RA, SZB = BN * RB;
  static constexpr int SZSA = SCALED ? BM * 4 : 0, SZSB = SCALED ? BN * 4 : 0;
  static constexpr int STAGE = SZA + SZB + SZSA + SZSB;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int NQA = SZA / 1024, NQB = SZB / 1024;  // 1 KiB wave copies per slice
  static constexpr int NW = WM * WN, NTHR = NW * 64;         // waves, threads per workgroup
  // bias / activation / 16-bit output in the epilogue: with 64 accumulator
  // fragments per lane (256 x 256 tiles) that code would not fit beside
  // them, so the launcher sends such epilogues to the 128 x 128 tiles
  static constexpr bool EPI_GENERAL = FM * FN <= 16;
  static_assert(NQA % NW == 0 && NQB % NW == 0, "tile copies split evenly over the waves");
  static_assert(BM <= NTHR && BN <= NTHR, "one scale row per thread");
  static_assert(!(BKN && KIND != kF16), "K x N right operand only for fp16");
  static_assert(!B6 || (KIND == kMX && FA == kFmtFp8 && (BM == 128 || BM == 256)),
                "FP6 weights: E4M3 x FP6 on 128 x 128 or 256 x 256 tiles");
  static_assert(!(BI4 || BI2) || (KIND == kMX && FA == kFmtFp8 && (BM == 128 || BM == 256)),
                "integer weights: E4M3 x INT4 / INT2 on 128 x 128 or 256 x 256 tiles");
};

struct Args {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  Epi e;                // output: C, bias, activation, element type
  int M, N, K;
  int tiles_m, tiles_n;
  int64_t lda, ldb;     // row strides in bytes of A and B (B: of its K x N rows when BKN)
  int nsteps;           // slices, the last one possibly partial
  int tail_a, tail_b;   // valid bytes per row in the last slice (== RA/RB when full)
  int scale_aligned;    // scale rows are 4-byte aligned and K % 128 == 0
};

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <class T>
struct Kernel {
  // ---- copy of one operand slice: BM rows x R bytes, direct to LDS --------
  template <int R, int NQ>
  static __device__ __forceinline__ void issue_rows(const uint8_t* __restrict__ g, int64_t ld, int row0,
                                                    int rows_valid, int64_t col_byte, uint8_t* lds, int wave,
                                                    int lane) {
#pragma unroll
    for (int t = 0; t < NQ / T::NW; t++) {
      const int q = wave + T::NW * t;
      const int o = q * 1024 + lane * 16;
      const int row = o / R;
      const int pch = (o % R) >> 4;
      const int c = pch ^ (R == 128 ? swz8(row) : R == 64 ? swz4(row) : 0);  // 32-byte rows: 2 chunks, none
      const int grow = min(row0 + row, rows_valid - 1);
      // a chunk reaching past the end of the row (partial last slice) reads
      // the slice's first chunk instead, which is always in bounds; it is
      // zeroed before use
      const int cc = (col_byte + c * 16 + 16 <= ld) ? c : 0;
      copy16_to_lds(g + (int64_t)grow * ld + col_byte + cc * 16, lds + q * 1024);
    }
  }
  // FP6 rows (K a multiple of 128, so every slice is whole): piece p (12
  // bytes, k 16 p .. 16 p + 15 of the slice) of row r lands in the 16-byte
  // slot p ^ swz8(r) of the 128-byte LDS row (a 12-byte copy writes lane l at
  // 16 l; the slot's last 4 bytes stay unwritten)
  template <int NQ>
  static __device__ __forceinline__ void issue_rows6(const uint8_t* __restrict__ g, int64_t ld, int row0,
                                                     int rows_valid, int64_t col_byte, uint8_t* lds, int wave,
                                                     int lane) {
    constexpr int kRsrcWord3 = 0x00020000;
    const int nrows = min(rows_valid - row0, T::BN);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc((void*)(g + (int64_t)row0 * ld), 0, (int)(nrows * ld),
                                                      kRsrcWord3);
#pragma unroll
    for (int t = 0; t < NQ / T::NW; t++) {
      const int q = wave + T::NW * t;
      const int o = q * 1024 + lane * 16;
      const int row = o / 128;
      const int c = ((o % 128) >> 4) ^ swz8(row);
      const int grow = min(row, nrows - 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + q * 1024), 12,
                                               (uint32_t)((int64_t)grow * ld + col_byte + c * 12), 0, 0, 0);
    }
  }
  // In a partial last slice, chunks past K were copied from in-bounds but
  // meaningless bytes; each lane overwrites the chunks it copied with zeros.
  template <int R, int NQ>
  static __device__ __forceinline__ void zero_tail(int valid_bytes, uint8_t* lds, int wave, int lane) {
#pragma unroll
    for (int t = 0; t < NQ / T::NW; t++) {
      const int q = wave + T::NW * t;
      const int o = q * 1024 + lane * 16;
      const int row = o / R;
      const int pch = (o % R) >> 4;
      const int c = pch ^ (R == 128 ? swz8(row) : R == 64 ? swz4(row) : 0);  // 32-byte rows: 2 chunks, none
      if (c * 16 >= valid_bytes) *reinterpret_cast<v4i*>(lds + o) = v4i{0, 0, 0, 0};
    }
  }
  // ---- scale bytes of one slice: 4 per row, through a register -----------
  static __device__ __forceinline__ uint32_t load_scales(const uint8_t* __restrict__ s, int rows_valid, int row0,
                                                         int nrows, int tid, int K, int step, bool aligned) {
    if (tid >= nrows) return 0u;
    const int grow = min(row0 + tid, rows_valid - 1);
    const int nb = K >> 5;
    const uint8_t* p = s + (int64_t)grow * nb + step * 4;
    if (aligned) return *reinterpret_cast<const uint32_t*>(p);
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t b = (step * 4 + i < nb) ? (uint32_t)p[i] : 127u;  // pad blocks: 2^0 times zero codes
      v |= b << (8 * i);
    }
    return v;
  }

  // ---- fp16 right operand stored K x N: register transpose into N x K ----
  struct KNRegs {
    v4i v[(16 * (T::BN / 8) + T::NTHR - 1) / T::NTHR][4];
  };
  static __device__ __forceinline__ void load_kn(const Args& a, int n0, int step, int tid, KNRegs& r) {
    // blocks of 4 (k) x 8 (n) halves; 16 * BN/8 blocks per slice
    constexpr int NBLK = 16 * (T::BN / 8);
    const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B);
#pragma unroll
    for (int j = 0; j < (NBLK + T::NTHR - 1) / T::NTHR; j++) {
      const int blk = tid + T::NTHR * j;
      if (blk >= NBLK) break;
      const int kb4 = blk & 15, nb8 = blk >> 4;
      const int n = n0 + nb8 * 8;
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        const int k = step * 64 + kb4 * 4 + kk;
        v4i val = {0, 0, 0, 0};
        if (k < a.K) {
          const uint16_t* row = B + (int64_t)k * a.N;
          if (n + 7 < a.N && (a.N & 7) == 0) {
            val = *reinterpret_cast<const v4i*>(row + n);
          } else {
            uint16_t h[8];
#pragma unroll
            for (int t = 0; t < 8; t++) h[t] = (n + t < a.N) ? row[n + t] : (uint16_t)0;
#pragma unroll
            for (int t = 0; t < 4; t++) val[t] = (int)((uint32_t)h[2 * t] | ((uint32_t)h[2 * t + 1] << 16));
          }
        }
        r.v[j][kk] = val;
      }
    }
  }
  static __device__ __forceinline__ void commit_kn(const KNRegs& r, uint8_t* ldsB, int tid) {
    constexpr int NBLK = 16 * (T::BN / 8);
#pragma unroll
    for (int j = 0; j < (NBLK + T::NTHR - 1) / T::NTHR; j++) {
      const int blk = tid + T::NTHR * j;
      if (blk >= NBLK) break;
      const int kb4 = blk & 15, nb8 = blk >> 4;
#pragma unroll
      for (int t = 0; t < 8; t++) {
        // column t of the 4 x 8 block: halves (k0..k0+3, n = nb8*8 + t)
        uint32_t h[4];
#pragma unroll
        for (int kk = 0; kk < 4; kk++) {
          const uint32_t w = (uint32_t)r.v[j][kk][t >> 1];
          h[kk] = (t & 1) ? (w >> 16) : (w & 0xffffu);
        }
        const int row = nb8 * 8 + t;
        const int chunk = kb4 >> 1;
        const int off = row * 128 + ((chunk ^ swz8(row)) << 4) + (kb4 & 1) * 8;
        *reinterpret_cast<v2i*>(ldsB + off) = v2i{(int)(h[0] | (h[1] << 16)), (int)(h[2] | (h[3] << 16))};
      }
    }
  }

  // ---- fragment reads ------------------------------------------------------
  // fp8 / fp16 rows: chunks g and 4 + g; fp4 rows: chunk g.
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

  // FP6 operand of row `row`: lane group g holds k 32 g .. 32 g + 31, the
  // pieces 2 g and 2 g + 1 (12 bytes each)
  static __device__ __forceinline__ v8i read_frag6(const uint8_t* lds, int row, int g) {
    const int s = swz8(row);
    const v4i lo = *reinterpret_cast<const v4i*>(lds + row * 128 + (((2 * g) ^ s) << 4));
    const v4i hi = *reinterpret_cast<const v4i*>(lds + row * 128 + (((2 * g + 1) ^ s) << 4));
    return v8i{lo[0], lo[1], lo[2], hi[0], hi[1], hi[2], 0, 0};
  }
  // INT4 operand of row `row` remapped to E4M3 codes: the fp8 operand's k
  // ranges 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15 are the 8 code
  // bytes at 8 g and 32 + 8 g of the 64-byte row (16-byte chunks swizzled by
  // swz4)
  static __device__ __forceinline__ v8i read_frag_int4(const uint8_t* lds, int row, int g) {
    const int s = swz4(row);
    const v2i lo = *reinterpret_cast<const v2i*>(lds + row * 64 + (((g >> 1) ^ s) << 4) + 8 * (g & 1));
    const v2i hi = *reinterpret_cast<const v2i*>(lds + row * 64 + (((2 + (g >> 1)) ^ s) << 4) + 8 * (g & 1));
    uint32_t e[8];
    int4x8_to_e4m3((uint32_t)lo[0], e[0], e[1]);
    int4x8_to_e4m3((uint32_t)lo[1], e[2], e[3]);
    int4x8_to_e4m3((uint32_t)hi[0], e[4], e[5]);
    int4x8_to_e4m3((uint32_t)hi[1], e[6], e[7]);
    return v8i{(int)e[0], (int)e[1], (int)e[2], (int)e[3], (int)e[4], (int)e[5], (int)e[6], (int)e[7]};
  }
  // INT2 operand of row `row` remapped to E2M1 codes: the fp4 operand's k
  // range 32 g .. 32 g + 31 is the 8 code bytes at 8 g of the 32-byte row
  static __device__ __forceinline__ v8i read_frag_int2(const uint8_t* lds, int row, int g) {
    const v2i c = *reinterpret_cast<const v2i*>(lds + row * 32 + 8 * g);
    uint32_t e[4];
    int2x16_to_e2m1((uint32_t)c[0], e[0], e[1]);
    int2x16_to_e2m1((uint32_t)c[1], e[2], e[3]);
    return v8i{(int)e[0], (int)e[1], (int)e[2], (int)e[3], 0, 0, 0, 0};
  }
  template <bool SIX>
  static __device__ __forceinline__ v8i read_b(const uint8_t* lds, int row, int g) {
    if constexpr (SIX)
      return read_frag6(lds, row, g);
    else if constexpr (T::BI4)
      return read_frag_int4(lds, row, g);
    else if constexpr (T::BI2)
      return read_frag_int2(lds, row, g);
    else
      return read_frag<T::RB>(lds, row, g);
  }

  // E4M3 byte pair -> two fp16 values times 2^(scale-127), rounded to fp16.
  static __device__ __forceinline__ uint32_t deq_pair(uint32_t two, uint32_t sbyte) {
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const uint32_t c = (two >> (8 * i)) & 0xffu;
      // s.eeee.mmm << 7 is the binary16 pattern of (E4M3 value) * 2^-8,
      // subnormals included
      const uint16_t hb = (uint16_t)(((c & 0x80u) << 8) | ((c & 0x7fu) << 7));
      float v = (float)__builtin_bit_cast(_Float16, hb);
      v = __builtin_ldexpf(v, (int)sbyte - 119);
      if ((c & 0x7fu) == 0x7fu || sbyte == 255u) v = __builtin_nanf("");
      const _Float16 h = (_Float16)v;
      out |= (uint32_t)__builtin_bit_cast(uint16_t, h) << (16 * i);
    }
    return out;
  }
  // 32 E4M3 codes of one lane (two 16-byte chunks) -> 4 x 8 fp16 values;
  // chunk 0 belongs to block g/2, chunk 1 to block 2 + g/2 of the slice.
  static __device__ __forceinline__ void deq_frag(const v8i& f, uint32_t sdw, int g, v8h out[4]) {
    const uint32_t s0 = (sdw >> (8 * (g >> 1))) & 0xffu;
    const uint32_t s1 = (sdw >> (8 * (2 + (g >> 1)))) & 0xffu;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint32_t sb = (q < 2) ? s0 : s1;
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const uint32_t word = (uint32_t)f[2 * q + t];
        w[2 * t] = deq_pair(word & 0xffffu, sb);
        w[2 * t + 1] = deq_pair(word >> 16, sb);
      }
      out[q] = __builtin_bit_cast(v8h, v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]});
    }
  }

  static __device__ __forceinline__ void run(const Args& a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int wi = wave / T::WN, wj = wave % T::WN;
    int tm, tn;
    tile_of_block(blockIdx.x, a.tiles_m, a.tiles_n, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;

    v4f acc[T::FM][T::FN];
#pragma unroll
    for (int i = 0; i < T::FM; i++)
#pragma unroll
      for (int j = 0; j < T::FN; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    uint32_t sa_reg = 0, sb_reg = 0;
    KNRegs kn;

    auto stage_ptr = [&](int st) { return smem + st * T::STAGE; };
    auto issue = [&](int step, int st) {
      uint8_t* base = stage_ptr(st);
      issue_rows<T::RA, T::NQA>(a.A, a.lda, m0, a.M, (int64_t)step * T::RA, base, wave, lane);
      if (T::BKN)
        load_kn(a, n0, step, tid, kn);
      else if constexpr (T::B6)
        issue_rows6<T::NQB>(a.B, a.ldb, n0, a.N, (int64_t)step * 96, base + T::SZA, wave, lane);
      else
        issue_rows<T::RB, T::NQB>(a.B, a.ldb, n0, a.N, (int64_t)step * T::RB, base + T::SZA, wave, lane);
      if (T::SCALED) {
        sa_reg = load_scales(a.SA, a.M, m0, T::BM, tid, a.K, step, a.scale_aligned);
        sb_reg = load_scales(a.SB, a.N, n0, T::BN, tid, a.K, step, a.scale_aligned);
      }
    };
    auto commit = [&](int step, int st) {
      uint8_t* base = stage_ptr(st);
      if (step == a.nsteps - 1) {
        if (a.tail_a < T::RA) zero_tail<T::RA, T::NQA>(a.tail_a, base, wave, lane);
        if (!T::BKN && !T::B6 && a.tail_b < T::RB) zero_tail<T::RB, T::NQB>(a.tail_b, base + T::SZA, wave, lane);
      }
      if (T::BKN) commit_kn(kn, base + T::SZA, tid);
      if (T::SCALED) {
        if (tid < T::BM) reinterpret_cast<uint32_t*>(base + T::SZA + T::SZB)[tid] = sa_reg;
        if (tid < T::BN) reinterpret_cast<uint32_t*>(base + T::SZA + T::SZB + T::SZSA)[tid] = sb_reg;
      }
    };

    if constexpr (T::KIND_ == kMX) mfma_fence_init(acc);
    issue(0, 0);
    for (int step = 0; step < a.nsteps; step++) {
      const int st = step & 1;
      wait_vmem();
      commit(step, st);
      __syncthreads();
      if (step + 1 < a.nsteps) issue(step + 1, st ^ 1);

      const uint8_t* la = stage_ptr(st);
      const uint8_t* lb = la + T::SZA;
      const uint32_t* lsa = reinterpret_cast<const uint32_t*>(lb + T::SZB);
      const uint32_t* lsb = lsa + T::BM;

      if constexpr (T::KIND_ == kMX) {
        // all A fragments stay in registers; B fragments stream through a
        // two-deep register buffer, one B column block per group of FM MFMAs
        // Scale bytes are read from LDS one byte each, straight into the
        // MFMA's scale registers: a VALU instruction (a shift) writing them
        // would need wait states before the inline MFMA reads them.
        const uint8_t* lsa8 = reinterpret_cast<const uint8_t*>(lsa);
        const uint8_t* lsb8 = reinterpret_cast<const uint8_t*>(lsb);
        v8i af[T::FM];
        int sa[T::FM];
#pragma unroll
        for (int i = 0; i < T::FM; i++) {
          const int row = wi * T::TM + i * 16 + r;
          af[i] = read_frag<T::RA>(la, row, g);
          sa[i] = lsa8[row * 4 + g];
        }
        v8i bcur = read_b<T::B6>(lb, wj * T::TN + r, g);
        int sbcur = lsb8[(wj * T::TN + r) * 4 + g];
#pragma unroll
        for (int j = 0; j < T::FN; j++) {
          v8i bnext = bcur;
          int sbnext = sbcur;
          if (j + 1 < T::FN) {
            const int row = wj * T::TN + (j + 1) * 16 + r;
            bnext = read_b<T::B6>(lb, row, g);
            sbnext = lsb8[row * 4 + g];
          }
#pragma unroll
          for (int i = 0; i < T::FM; i++)
            if constexpr (T::BI4)
              mfma_scaled_acc_after_valu(acc[i][j], bcur, af[i], sbcur, sa[i]);
            else if constexpr (T::BI2)
              mfma_scaled_acc_fp4a_after_valu(acc[i][j], bcur, af[i], sbcur, sa[i]);
            else
              mfma_scaled_acc<T::FBM, T::FA>(acc[i][j], bcur, af[i], sbcur, sa[i]);
          bcur = bnext;
          sbcur = sbnext;
        }
      } else if constexpr (T::KIND_ == kF16) {
        v8i af[T::FM], bf[T::FN];
#pragma unroll
        for (int i = 0; i < T::FM; i++) af[i] = read_frag<128>(la, wi * T::TM + i * 16 + r, g);
#pragma unroll
        for (int j = 0; j < T::FN; j++) bf[j] = read_frag<128>(lb, wj * T::TN + j * 16 + r, g);
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
          for (int i = 0; i < T::FM; i++)
#pragma unroll
            for (int j = 0; j < T::FN; j++) {
              const v4i bq = h ? v4i{bf[j][4], bf[j][5], bf[j][6], bf[j][7]} : v4i{bf[j][0], bf[j][1], bf[j][2], bf[j][3]};
              const v4i aq = h ? v4i{af[i][4], af[i][5], af[i][6], af[i][7]} : v4i{af[i][0], af[i][1], af[i][2], af[i][3]};
              acc[i][j] = mfma_f16_16x16x32(__builtin_bit_cast(v8h, bq), __builtin_bit_cast(v8h, aq), acc[i][j]);
            }
      } else {  // kDEQ
        v8h ah[T::FM][4], bh[T::FN][4];
#pragma unroll
        for (int i = 0; i < T::FM; i++) {
          const int row = wi * T::TM + i * 16 + r;
          deq_frag(read_frag<128>(la, row, g), lsa[row], g, ah[i]);
        }
#pragma unroll
        for (int j = 0; j < T::FN; j++) {
          const int row = wj * T::TN + j * 16 + r;
          deq_frag(read_frag<128>(lb, row, g), lsb[row], g, bh[j]);
        }
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int i = 0; i < T::FM; i++)
#pragma unroll
            for (int j = 0; j < T::FN; j++) acc[i][j] = mfma_f16_16x16x32(bh[j][q], ah[i][q], acc[i][j]);
      }
    }

    if constexpr (T::KIND_ == kMX) mfma_drain(acc);

    // ---- epilogue: lane (g, r) holds C[m][n .. n+3] -------------------------
    const bool vec_ok = (a.N & 3) == 0;
    const Epi e = T::EPI_GENERAL ? a.e : Epi{a.e.C, nullptr, kOutF32, kActNone};
#pragma unroll
    for (int i = 0; i < T::FM; i++) {
      const int m = m0 + wi * T::TM + i * 16 + r;
      if (m >= a.M) continue;
#pragma unroll
      for (int j = 0; j < T::FN; j++) {
        const int n = n0 + wj * T::TN + j * 16 + 4 * g;
        epi_store4<false>(e, a.N, m, n, acc[i][j], vec_ok && n + 3 < a.N);
      }
    }
  }
};

template <class T, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(T::NTHR, T::NTHR),
                          amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void tiled_kernel(Args a) {
  Kernel<T>::run(a);
}

template <class T, int WPE>
hipError_t launch(const Args& a0, hipStream_t stream) {
  Args a = a0;
  a.tiles_m = (a.M + T::BM - 1) / T::BM;
  a.tiles_n = (a.N + T::BN - 1) / T::BN;
  a.nsteps = (a.K + T::KSLICE - 1) / T::KSLICE;
  const int rem = a.K - (a.nsteps - 1) * T::KSLICE;  // K elements in the last slice
  auto bytes = [&](bool f4, bool f16, int elems) { return f16 ? elems * 2 : (f4 ? elems / 2 : elems); };
  a.tail_a = bytes(T::AF4, !T::SCALED, rem);
  a.tail_b = T::BI2 ? rem / 4 : bytes(T::BF4 || T::BI4, !T::SCALED, rem);
  const int64_t nt = (int64_t)a.tiles_m * a.tiles_n;
  hipLaunchKernelGGL((tiled_kernel<T, WPE>), dim3((unsigned)nt), dim3(T::NTHR), 0, stream, a);
  return hipGetLastError();
}

Args make_args(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e, int64_t M,
               int64_t N, int64_t K) {
  Args a{};
  a.A = (const uint8_t*)A;
  a.SA = SA;
  a.B = (const uint8_t*)B;
  a.SB = SB;
  a.e = e;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  return a;
}

// Configurations: 256 x 256 tiles (one workgroup per CU, 128 x 128 per wave)
// for large outputs, 128 x 128 (two workgroups per CU) otherwise.
template <int FA, int FB>
using MxBig = Cfg<kMX, 256, 256, 2, 2, FA, FB, false>;
template <int FA, int FB>
using MxMid = Cfg<kMX, 128, 128, 2, 2, FA, FB, false>;
// integer weights: 1 x 4 waves (128 x 32 per wave), so that each B fragment
// is read and remapped by one wave only, where 2 x 2 waves remap every one
// twice (measured at 8192 x 14336 x 4096: INT4 0.778 -> 0.695 ms, INT2 0.626
// -> 0.595 ms; FP6 weights, whose fragments are only gathered, gained
// nothing and keep 2 x 2).  Outputs of at least 256 tiles of 256 x 256 with
// a plain fp32 store take the 256 x 256 tiles (2 x 2 waves of 128 x 128:
// each fragment is remapped or gathered by two waves but feeds 8 MFMAs in
// each, with fewer LDS bytes per MFMA; INT4 0.685 -> 0.665 ms, INT2 0.585 ->
// 0.556 ms, FP6 0.685 -> 0.605 ms)
template <int FB>
using MxIntMid = Cfg<kMX, 128, 128, 1, 4, kFmtFp8, FB, false>;
using MxBig88 = MxBig<kFmtFp8, kFmtFp8>;
using MxMid88 = MxMid<kFmtFp8, kFmtFp8>;
using MxMid84 = MxMid<kFmtFp8, kFmtFp4>;
using MxMid44 = MxMid<kFmtFp4, kFmtFp4>;
using F16Big = Cfg<kF16, 256, 256, 2, 2, kFmtFp8, kFmtFp8, false>;
using F16Mid = Cfg<kF16, 128, 128, 2, 2, kFmtFp8, kFmtFp8, false>;
using F16MidKN = Cfg<kF16, 128, 128, 2, 2, kFmtFp8, kFmtFp8, true>;
// K x N right operand with fewer 128 x 128 tiles than CUs: 64 x 64 tiles
using F16SmallKN = Cfg<kF16, 64, 64, 2, 2, kFmtFp8, kFmtFp8, true>;
using DeqMid = Cfg<kDEQ, 128, 128, 2, 2, kFmtFp8, kFmtFp8, false>;

template <int FA, int FB>
hipError_t launch_mx_fmt(const Args& a, bool big, hipStream_t stream) {
  return big ? launch<MxBig<FA, FB>, 1>(a, stream) : launch<MxMid<FA, FB>, 2>(a, stream);
}

bool use_big_tiles(int64_t M, int64_t N) {
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  return big_tiles >= 256;
}

}  // namespace

hipError_t launch_mx_tiled(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                           int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream) {
  Args a = make_args(A, SA, B, SB, e, M, N, K);
  const bool af4 = (fmt == 2), bf4 = (fmt == 1 || fmt == 2 || fmt == 6), bf6 = (fmt == 8 || fmt == 9);
  a.lda = af4 ? K / 2 : K;
  a.ldb = bf4 ? K / 2 : bf6 ? K / 4 * 3 : fmt == 7 ? K / 4 : K;
  a.scale_aligned = ((K & 127) == 0 && ((uintptr_t)SA & 3) == 0 && ((uintptr_t)SB & 3) == 0) ? 1 : 0;
  // E4M3 x FP6 (K a multiple of 128, checked by the caller): 128 x 128 tiles
  const bool big_int = use_big_tiles(M, N) && e.bias == nullptr && e.act == kActNone && e.out == kOutF32;
  if (fmt == 8) return big_int ? launch<MxBig<kFmtFp8, kFmtFp6>, 1>(a, stream) : launch<MxMid<kFmtFp8, kFmtFp6>, 2>(a, stream);
  if (fmt == 9) return big_int ? launch<MxBig<kFmtFp8, kFmtBf6>, 1>(a, stream) : launch<MxMid<kFmtFp8, kFmtBf6>, 2>(a, stream);
  // E4M3 x INT4 (codes remapped to E4M3 in registers): 128 x 128 tiles
  if (fmt == 6) return big_int ? launch<MxBig<kFmtFp8, kElemInt4>, 1>(a, stream) : launch<MxIntMid<kElemInt4>, 2>(a, stream);
  // E4M3 x INT2 (codes remapped to E2M1 in registers): 128 x 128 tiles
  if (fmt == 7) return big_int ? launch<MxBig<kFmtFp8, kElemInt2>, 1>(a, stream) : launch<MxIntMid<kElemInt2>, 2>(a, stream);
  // the 256 x 256 tiled kernels store plain fp32 only (MxBig*::EPI_GENERAL)
  const bool big_pp = use_big_tiles(M, N);
  if (big_pp && pingpong_mx_ok(SA, SB, M, N, K)) return launch_mx_pingpong(A, SA, B, SB, e, M, N, K, fmt, stream);
  if (pp128_mx_ok(SA, SB, M, N, K)) return launch_mx_pp128(A, SA, B, SB, e, M, N, K, fmt, stream);
  const bool big = big_pp && e.bias == nullptr && e.act == kActNone && e.out == kOutF32;
  static_assert(!MxBig88::EPI_GENERAL && MxMid88::EPI_GENERAL && MxMid84::EPI_GENERAL && MxMid44::EPI_GENERAL,
                "general epilogues run on the 128 x 128 tiles");
  switch (fmt) {
    case 0: return launch_mx_fmt<kFmtFp8, kFmtFp8>(a, big, stream);
    case 1: return launch_mx_fmt<kFmtFp8, kFmtFp4>(a, big, stream);
    case 2: return launch_mx_fmt<kFmtFp4, kFmtFp4>(a, big, stream);
    case 3: return launch_mx_fmt<kFmtBf8, kFmtBf8>(a, big, stream);
    case 4: return launch_mx_fmt<kFmtFp8, kFmtBf8>(a, big, stream);
    default: return launch_mx_fmt<kFmtBf8, kFmtFp8>(a, big, stream);
  }
}

hipError_t launch_f16_tiled(const uint16_t* A, const uint16_t* B, float* C, int64_t M, int64_t N, int64_t K,
                            int b_is_nk, hipStream_t stream) {
  Args a = make_args(A, nullptr, B, nullptr, Epi{C, nullptr, kOutF32, kActNone}, M, N, K);
  a.lda = K * 2;
  if (!b_is_nk) {
    a.ldb = N * 2;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 256;
    if (((M + 127) / 128) * ((N + 127) / 128) < cus) return launch<F16SmallKN, 2>(a, stream);
    return launch<F16MidKN, 2>(a, stream);
  }
  a.ldb = K * 2;
  if (use_big_tiles(M, N) && M % 256 == 0 && N % 256 == 0 && K % 64 == 0) return launch_f16_pingpong(A, B, C, M, N, K, stream);
  if (M % 128 == 0 && N % 128 == 0 && K % 64 == 0) return launch_f16_pp128(A, B, C, M, N, K, stream);
  return use_big_tiles(M, N) ? launch<F16Big, 1>(a, stream) : launch<F16Mid, 2>(a, stream);
}

hipError_t launch_deq_tiled(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, float* C, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream) {
  Args a = make_args(A, SA, B, SB, Epi{C, nullptr, kOutF32, kActNone}, M, N, K);
  a.lda = K;
  a.ldb = K;
  a.scale_aligned = ((K & 127) == 0 && ((uintptr_t)SA & 3) == 0 && ((uintptr_t)SB & 3) == 0) ? 1 : 0;
  return launch<DeqMid, 2>(a, stream);
}

}  // namespace mxg
