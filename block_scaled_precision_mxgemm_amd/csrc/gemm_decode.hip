// gemm_decode.hip - MX GEMM for decode shapes with few activation rows (M <= 64)
// against a large weight matrix B (N x K: E4M3, E2M1, E2M3, E3M2, INT4 or INT2
// elements with UE8M0 block scales; K a multiple of 1024 from 2048; one
// launch takes up to 12288 of it with 8- and 6-bit weights, 14336 with INT4
// and 16384 with E2M1 and INT2 ones, longer K runs in chunks that add into an
// fp32 C).  The
// product is bound by the bytes of B, which must stream from HBM exactly
// once; the weight plane is what quantization shrinks ("Metal tensors で
// カスタム機械学習オペレーションを最適化する", section "主要内容": inference
// is memory-bandwidth bound and quantization cuts both the footprint and the
// traffic).
//
// Design (gfx950):
//   * one persistent workgroup of 8 waves per CU owns a contiguous range of
//     16-row blocks of B ("fragments");
//   * wave w owns the k range [w K/8, (w+1) K/8) of every fragment (but see
//     the uneven split below) and holds
//     the matching A operands (1 to 4 blocks of 16 rows) in registers for the
//     whole kernel; each weight operand it reads from LDS feeds one MFMA per
//     row block;
//   * each wave streams its own k band of the fragment rows through a private
//     LDS ring of stages (16 rows x 128 bytes) with direct global->LDS copies
//     of 8 rows x 128 bytes per instruction (whole cache lines; this pattern
//     streams as fast as 1 KiB row segments on MI355X, 5.7 TB/s for a
//     112 MiB read).  A wave waits only for its own copies: the stages need
//     no workgroup barrier.  With MXFP4 weights and K / 1024 odd, one eighth
//     of a row is an odd number of 64-byte MFMA operands; waves 0-3 then take
//     one operand more and waves 4-7 one less, so every band is whole
//     128-byte stages;
//   * inside a 128-byte stage row the 16-byte chunks are XOR-swizzled with
//     (row >> 1) & 7 (applied on the global side, so the copy still writes LDS
//     linearly), which makes the MFMA fragment reads conflict-free;
//   * a fragment's 8 per-wave partial sums meet in LDS after one barrier per
//     fragment; one wave per 16-row block adds them in a fixed order, so the
//     result is deterministic and needs no atomics, and keeps the sum in
//     registers: C is stored after the stream.
#include <utility>

#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

constexpr int kDecWaves = 8;
// Per-wave ring depth (a power of two): 3 stages in flight per wave (48 KiB
// per CU) keep HBM as busy as 7 do, and the shallower first burst of copies
// brings each wave's first stage back sooner (16 x 28672 x 8192: 24.3 us at
// depth 4 against 25.7 us at depth 8; fp8 weights 39.7 against 39.4 us).
// Operands of 64 bytes or less and FP6 line stages keep 2 stages in flight
// in this ring (Decode::AHEAD).
constexpr int kDecStages = 4;
// Ring depth when every workgroup owns at most one fragment (N <= 16 x CUs):
// a wave's whole stream is then a few stages, all of which can be in flight
// at once (16 x 4096 x 4096 fp8 x fp4: 9.8 against 11.0 us; 8 x 2048 x 8192:
// 9.6-9.8 against 10.7 us; allowing 2 or 4 fragments per workgroup made
// 16 x 8192 x 8192 slower, 13.6-13.8 against 12.2 us).
constexpr int kDecStagesDeep = 8;
constexpr int kDeepMaxFrags = 1;
constexpr int kBand = 128;                    // bytes of each weight row per stage and wave
constexpr int kStageBytes = 16 * kBand;       // one stage: 16 rows
// FP6 weights: one 96-byte MFMA operand per row and stage, copied 12 bytes
// per lane; the copy writes lane l at 16 l of LDS (the slot's last 4 bytes
// are not written), so a stage keeps the 128-byte rows of the other formats
// with 12-byte pieces in 16-byte slots, swizzled the same way
constexpr bool is_fp6(int w) { return w == kFmtFp6 || w == kFmtBf6; }
// FP6 weights with K / 1024 a multiple of 4 instead stream whole 128-byte
// lines per row and stage (16-byte copies, as for the other formats): a
// wave's band is then 3 K / 4096 stages holding 4 operands per 3 stages, and
// an operand may begin in the stage before the one that completes it
constexpr bool fp6_line(int w, int kw) { return is_fp6(w) && kw % 4 == 0; }
constexpr int band_bytes(int w, int kw) { return is_fp6(w) && !fp6_line(w, kw) ? 96 : kBand; }  // global bytes of a row per stage
// Reduced output blocks (16 x 16) a wave keeps in registers until its
// copies are done.  A store issued inside the stream would sit among the copies in the
// in-order vector-memory counter and make the next stage waits of that wave
// also wait for the store and for one more stage; with the barrier per
// fragment every wave would then lose that time.
constexpr int kHeld = 4;
// Cache policy of the weight and weight-scale copies: non-temporal (the
// "nt" bit of gfx950 buffer loads).  The weights are read exactly once, and
// streaming them without normal cache retention measured 4 % faster for fp4
// and 7 % faster for fp8 weights on the 16 x 28672 x 8192 decode shape.
constexpr int kStreamPolicy = 2;

struct DecArgs {
  const uint8_t* A;   // at this launch's first row and K chunk
  const uint8_t* SA;
  const uint8_t* B;   // at this launch's K chunk
  const uint8_t* SB;
  Epi e;       // output: C (this launch's first row), bias, activation, element type
  int M, N, K; // K: this launch's chunk of the reduction
  int ldk;     // the whole K: the row strides of A, B and the scale planes follow it
  int accum;   // 1: fp32 C already holds the sum over earlier K chunks; add to it
  int nfrags;  // ceil(N / 16)
};

__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Weight formats W: kFmtFp8 (E4M3, 128 bytes per 128-k MFMA operand),
// kFmtFp4 (E2M1, 64 bytes), kElemInt4 (64 bytes, remapped in registers to
// an E4M3 operand), kElemInt2 (32 bytes, remapped to an E2M1 operand),
// kFmtFp6 / kFmtBf6 (E2M3 / E3M2, 96 bytes, MFMA operands as stored).
constexpr int op_bytes(int w) { return w == kFmtFp8 ? 128 : is_fp6(w) ? 96 : w == kElemInt2 ? 32 : 64; }
// MFMA operand format the weights are fed as
constexpr int mfma_fmt(int w) {
  return is_fp6(w) ? w : (w == kFmtFp8 || w == kElemInt4) ? kFmtFp8 : kFmtFp4;
}
// stages per fragment of a wave with wk MFMAs
constexpr int stages_per_frag(int w, int wk) {
  return fp6_line(w, wk) ? 3 * wk / 4 : wk / (band_bytes(w, wk) / op_bytes(w));
}

// K / 1024 = KW MFMAs (128 k each) per wave per fragment on average.  With
// two MFMA operands per 128-byte stage (E2M1, INT4) and KW odd, waves 0-3
// take KW + 1 MFMAs and waves 4-7 KW - 1.  (INT2, four operands per stage,
// takes K / 1024 multiples of 4 only.)
constexpr bool split_k(int w, int kw) { return op_bytes(w) == 64 && kw % 2 == 1; }

// LDS of one wave's ring and scale slots for WK MFMAs per fragment
constexpr int ring_bytes(int w, int wk, int d) {
  const int nq = stages_per_frag(w, wk);
  const int nsi = (16 * wk + 63) / 64;
  const int nsl = (nq - 1 + d + nq - 1) / nq;
  return d * kStageBytes + nsl * nsi * 256;
}

// KW: K / 1024; XK: this wave's MFMAs per fragment are WK = KW + XK (XK = +1
// for waves 0-3 and -1 for waves 4-7 under the uneven split, else 0).  MB:
// blocks of 16 activation rows (M <= 16 MB); each weight operand read from
// LDS feeds one MFMA per block, so the weight stream is the same for every MB.
template <int W, int KW, int MB, int D_, int XK>
struct Decode {
  static constexpr int D = D_;
  static constexpr int WK = KW + XK;                     // MFMAs per fragment of this wave
  static constexpr int OPB = op_bytes(W);                // bytes of a weight row per MFMA
  static constexpr bool LINE = fp6_line(W, WK);          // FP6 operands across 128-byte line stages
  static constexpr int BAND = band_bytes(W, WK);         // global bytes of a weight row per stage
  static constexpr int STAGE = kStageBytes;              // one stage in LDS: 16 rows of 128 bytes
  static constexpr int MPS = LINE ? 1 : BAND / OPB;      // MFMAs per stage (accumulators)
  static constexpr int NQ = stages_per_frag(W, WK);      // stages per fragment
  static constexpr int CPB = is_fp6(W) && !LINE ? 12 : 16;  // bytes per lane of a weight copy
  // stages between a copy's issue and the stage that reads it: D - 1, and
  // D - 2 with line stages, whose straddling operands still read the
  // previous stage (the buffer then refilled is two stages old), and with
  // operands of 64 bytes or less in a 4-stage ring (16 x 28672 x 8192:
  // E2M1 23.50 -> 23.28 us, INT4 28.8 -> 28.6 us, INT2 19.75 -> 19.3 us;
  // E4M3 weights were 0.45 us slower that way)
  static constexpr int AHEAD = (LINE || (OPB <= 64 && D == 4)) ? D - 2 : D - 1;
  // MFMAs whose operands complete in stage q: ops_count(q) of them from
  // ops_first(q) (line stages: operand u ends at byte 96 u + 95 of the band)
  static constexpr int ops_first(int q) { return LINE ? 128 * q / 96 : q * MPS; }
  static constexpr int ops_count(int q) { return LINE ? (128 * q + 32) / 96 + 1 - ops_first(q) : MPS; }
  static constexpr int kBFmt = mfma_fmt(W);              // MFMA format of the weight operand
  static constexpr int SBW = 4 * WK;                     // scale bytes of a row per wave
  static constexpr int LPR = SBW / 4;                    // scale copy lanes per row (4 bytes each)
  static constexpr int NSI = (16 * LPR + 63) / 64;       // scale copies per fragment
  // scale slots: a fragment's slot is refilled only after its last stage
  static constexpr int NSL = (NQ - 1 + D + NQ - 1) / NQ;
  static constexpr int SZ_SC = NSI * 256;
  // every wave's region has the size of the larger wave kind's
  static constexpr int SZ_WAVE = XK == 0 ? ring_bytes(W, WK, D)
                                         : (ring_bytes(W, KW + 1, D) > ring_bytes(W, KW - 1, D)
                                                ? ring_bytes(W, KW + 1, D)
                                                : ring_bytes(W, KW - 1, D));
  static constexpr int OFF_PART = kDecWaves * SZ_WAVE;
  static constexpr int SZ_PSLOT = MB * kDecWaves * 64 * 16;  // one fragment's partials
  // Integer weights with one row block pass the fragment barrier every
  // second fragment (four partial-sum slots instead of two): 16 x 28672 x
  // 8192 INT4 29.9 -> 28.7 us, INT2 19.8 -> 19.6 us, identical results.
  // E2M1 weights measured 0.4 us slower that way, FP6 the same.
  static constexpr bool PAIRED = (W == kElemInt4 || W == kElemInt2) && MB == 1;
  static constexpr int NPSLOT = PAIRED ? 4 : 2;
  static constexpr int LDS = OFF_PART + NPSLOT * SZ_PSLOT;
  // loads of this wave's SBW = 4 KW A scale bytes per block: 16-byte loads,
  // then 8 and 4 bytes for the rest.  They are issued before any copy, so
  // the stage waits never count them (the compiler may merge the small ones).
  static constexpr int NS16 = SBW / 16, NS8 = (SBW % 16) / 8, NS4 = (SBW % 8) / 4;
  static constexpr bool FITS = LDS <= 160 * 1024;  // the 160 KiB LDS of a gfx950 CU
  static_assert(NQ >= 1 && (LINE ? WK % 4 == 0 && AHEAD >= 2 : WK % MPS == 0) && (D & (D - 1)) == 0,
                "whole stages per fragment");
  static_assert(ring_bytes(W, WK, D) == D * STAGE + NSL * SZ_SC && SZ_WAVE >= ring_bytes(W, WK, D),
                "region layout");
  static_assert(NSL * NQ >= NQ - 1 + D, "scale slot reuse");
  static_assert(MB >= 1 && MB * WK <= 16, "A operands of all blocks in 128 VGPRs");
  static_assert(XK == 0 || split_k(W, KW), "uneven split only for two operands per stage with K / 1024 odd");

  // first MFMA (128 k) of wave w's band: w KW, shifted by the uneven split
  static __device__ __forceinline__ int band_start(int w) { return w * KW + (XK > 0 ? w : XK < 0 ? 8 - w : 0); }

  // fp8 operand of the MFMA covering k0 .. k0+127 of row `p` (p at k0):
  // lane group g holds k0 + 16g .. +15 and k0 + 64 + 16g .. +15
  static __device__ __forceinline__ v8i load_fp8_op(const uint8_t* p, int g) {
    const v4i lo = *reinterpret_cast<const v4i*>(p + 16 * g);
    const v4i hi = *reinterpret_cast<const v4i*>(p + 64 + 16 * g);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }

  // Sum of the 8 per-wave partials of a fragment's row block mb, in wave
  // order.  Lane (g, r) holds C[16 mb + r][16 frag + 4g .. 4g+3].
  static __device__ __forceinline__ v4f reduce(const uint8_t* smem, int slot, int mb, int lane) {
    const v4f* part = reinterpret_cast<const v4f*>(smem + OFF_PART + slot * SZ_PSLOT) + mb * kDecWaves * 64;
    v4f s = part[lane];
#pragma unroll
    for (int w = 1; w < kDecWaves; w++) s += part[w * 64 + lane];
    return s;
  }

  static __device__ __forceinline__ void store_c(const DecArgs& a, int frag, int mb, v4f s, int g, int r) {
    const int m = 16 * mb + r;
    const int n = frag * 16 + 4 * g;
    if (m >= a.M) return;
    const bool vec = (a.N & 3) == 0 && n + 3 < a.N;
    if (a.accum) {
      const float* prev = reinterpret_cast<const float*>(a.e.C) + (int64_t)m * a.N + n;
      if (vec) {
        s += *reinterpret_cast<const v4f*>(prev);
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++)
          if (n + i < a.N) s[i] += prev[i];
      }
    }
    epi_store4<false>(a.e, a.N, m, n, s, vec);
  }

  // Per-wave state (all in registers once inlined).
  struct State {
    const DecArgs* a;
    uint8_t* smem;  // workgroup LDS
    uint8_t* wsm;   // this wave's ring and scale slots
    int lane, wave, g, r;
    int kb;               // this wave's first MFMA in a row: k = 128 kb
    int f_begin, nf;
    uint32_t rb, nb;      // bytes per B row, scale bytes per row
    int brow;             // lane's row in a copy of 8 rows
    uint32_t bch[2];      // lane's swizzled chunk offset, rows 0-7 / 8-15
    int srow[NSI];        // lane's row in each scale copy
    uint32_t scol[NSI];   // and its byte in that row's band
    v8i av[MB][WK];       // A operands of this wave's MFMAs, per row block
    uint32_t sa[MB][WK];  // their scale dwords (blocks 4j .. 4j+3); byte g is extracted at the MFMA
    v4f acc[MB][MPS];
    v4f held[kHeld];      // reduced blocks u = w, w + 8, ... (u = MB f + mb), stored at the end
  };

  // Vector-memory instructions of the A loads that stage q of the first
  // fragment needs (lo and hi halves per MFMA), and those of stages q ..
  // q + n - 1.  A(q) is issued right after stage q's copies: by the prologue
  // for q < AHEAD, else by stage q - AHEAD of the first fragment, so the
  // first stages' weights do not queue behind all of A (every CU reads the
  // same activations from L2 at the start: 16 x 28672 x 8192 E2M1 23.26 ->
  // 22.95 us, E4M3 39.6 -> 38.8, FP6 31.3 -> 30.6, INT4 28.4 -> 28.1 us
  // against all of A in the prologue; INT2 the same).
  static constexpr int la(int q) { return MB * 2 * ops_count(q); }
  static constexpr int la_range(int q, int n) { return (n <= 0 || q >= NQ) ? 0 : la(q) + la_range(q + 1, n - 1); }
  // Copies issued after stage s's copies and before its wait: the copies of
  // stages s+1 .. s+AHEAD-1 (2 weight copies each, plus the scale copies at
  // every fragment start) and, in the first fragment, the A loads of stages
  // q .. q+AHEAD-1, each issued right after that stage's copies.
  static constexpr int younger(int q, bool first) {
    return 2 * (AHEAD - 1) + NSI * ((q + AHEAD - 1) / NQ) + (first ? la_range(q, AHEAD) : 0);
  }

  template <int N>
  static __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
  }
  // the copies wait, plus every LDS access issued so far: the buffer and the
  // scale slot that the next copies refill were read at the previous stage
  template <int N>
  static __device__ __forceinline__ void wait_stage() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"i"(N) : "memory");
  }
  static __device__ __forceinline__ void order_fence() { asm volatile("" ::: "memory"); }

  // Copies of stage q of fragment fs.  fs may run past the workgroup's last
  // fragment.  In the prologue and the first fragment (fixed == true) the
  // last stage's source is then read again into a buffer no live stage uses:
  // the number of copies per stage stays fixed, so the compiler's own wait
  // counts for the A loads interleaved there stay exact.  Later such copies
  // are skipped (the stage waits then account for it).  Rows past N read row
  // N-1 again.  Every copy that is issued is issued by all lanes.
  // (q is a constant at every call site once inlined)
  static __device__ __forceinline__ void issue(State& t, int fs, int q, bool fixed) {
    constexpr int kRsrcWord3 = 0x00020000;
    const DecArgs& a = *t.a;
    if (!fixed && fs >= t.nf) return;
    const bool past = fs >= t.nf;
    const int fv = past ? t.nf - 1 : fs;
    const int qv = past ? NQ - 1 : q;
    const int row0 = (t.f_begin + fv) * 16;
    const int last = a.N - 1 - row0;
    if (q == 0) {
      const auto rs_s = __builtin_amdgcn_make_buffer_rsrc((void*)(a.SB + (int64_t)row0 * t.nb), 0, 16 * t.nb,
                                                          kRsrcWord3);
      uint8_t* sc = t.wsm + D * STAGE + (fs % NSL) * SZ_SC;
#pragma unroll
      for (int i = 0; i < NSI; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_s, (lds_void*)(sc + i * 256), 4,
                                                 (uint32_t)min(t.srow[i], last) * t.nb + t.scol[i],
                                                 (uint32_t)(4 * t.kb), 0, kStreamPolicy);
    }
    const auto rs_b = __builtin_amdgcn_make_buffer_rsrc((void*)(a.B + (int64_t)row0 * t.rb), 0, 16 * t.rb, kRsrcWord3);
    uint8_t* st = t.wsm + ((fs * NQ + q) & (D - 1)) * STAGE;
    const uint32_t soff = (uint32_t)(t.kb * OPB + qv * BAND);
#pragma unroll
    for (int h = 0; h < 2; h++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(st + h * 8 * kBand), CPB,
                                               (uint32_t)min(t.brow + 8 * h, last) * t.rb + t.bch[h], soff, 0,
                                               kStreamPolicy);
  }

  // A operands of the MFMAs of stage q of this wave (rows clamped to M-1;
  // rows >= M are computed and discarded): wave MFMA j covers k 128 (kb + j)
  // .. +127.
  template <int Q>
  static __device__ __forceinline__ void load_a(State& t) {
    const DecArgs& a = *t.a;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      const int m = min(16 * mb + t.r, a.M - 1);
      const uint8_t* row = a.A + (int64_t)m * a.ldk + (int64_t)t.kb * 128;
#pragma unroll
      for (int u = 0; u < ops_count(Q); u++)
        t.av[mb][ops_first(Q) + u] = load_fp8_op(row + (ops_first(Q) + u) * 128, t.g);
    }
  }

  // A scales of this wave: MFMA j takes byte g of the dword of blocks
  // 4 (kb + j) .. +3.  The dwords stay raw until the MFMA: extracting a byte
  // here would wait for these loads before the first copy is issued.
  static __device__ __forceinline__ void load_a_scales(State& t) {
    const DecArgs& a = *t.a;
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      const int m = min(16 * mb + t.r, a.M - 1);
      const uint8_t* srow = a.SA + (int64_t)m * t.nb + t.kb * 4;
#pragma unroll
      for (int i = 0; i < NS16; i++) {
        const v4i d = *reinterpret_cast<const v4i*>(srow + 16 * i);
#pragma unroll
        for (int e = 0; e < 4; e++) t.sa[mb][4 * i + e] = (uint32_t)d[e];
      }
      if constexpr (NS8 == 1) {
        const v2i d = *reinterpret_cast<const v2i*>(srow + 16 * NS16);
        t.sa[mb][4 * NS16] = (uint32_t)d[0];
        t.sa[mb][4 * NS16 + 1] = (uint32_t)d[1];
      }
      if constexpr (NS4 == 1) t.sa[mb][WK - 1] = *reinterpret_cast<const uint32_t*>(srow + SBW - 4);
    }
  }

  // Prologue, in this issue order: the A scales, then stage p's copies and
  // A(p), for p = 0 .. AHEAD - 1 (A(p) for p < NQ).
  template <int... P>
  static __device__ __forceinline__ void prologue(State& t, std::integer_sequence<int, P...>) {
    // an assembly comment naming the counted loads, for the static check of
    // the compiled code
    asm volatile("; decode prologue wk=%0 mb=%1 la=%2" ::"i"(WK), "i"(MB), "i"(la_range(0, AHEAD)));
    load_a_scales(t);
    order_fence();
    (
        [&] {
          if constexpr (P <= AHEAD - 1) issue(t, P / NQ, P % NQ, true);
          order_fence();
          if constexpr (P < NQ && P <= AHEAD - 1) load_a<P>(t);
          order_fence();
        }(),
        ...);
  }

  // Stage q of fragment f.
  template <int Q, bool FIRST>
  static __device__ __forceinline__ void stage(State& t, int f) {
    // this wave's copies of the stage are complete once at most the younger
    // vector-memory instructions are outstanding (the counter completes in
    // issue order; stores of C issued since are younger still and only make
    // the wait stricter).  Past the first fragment, when a younger stage lies
    // beyond the last one its copies were skipped, and the stage waits for
    // everything instead.
    if (FIRST || (f * NQ + Q) + AHEAD - 1 < t.nf * NQ)
      wait_stage<younger(Q, FIRST)>();
    else
      wait_stage<0>();
    // stage s + AHEAD, into the buffer read last at stage s - 1
    issue(t, f + (Q + AHEAD) / NQ, (Q + AHEAD) % NQ, FIRST);
    if constexpr (FIRST && Q + AHEAD < NQ) {
      // the A operands of stage Q + AHEAD, right after its copies
      order_fence();
      load_a<Q + AHEAD>(t);
      order_fence();
    }
    const uint8_t* st = t.wsm + ((f * NQ + Q) & (D - 1)) * STAGE;
    const uint8_t* sc = t.wsm + D * STAGE + (f % NSL) * SZ_SC;
    const int g = t.g, r = t.r;
    const int sw = (r >> 1) & 7;
#pragma unroll
    for (int u = 0; u < ops_count(Q); u++) {
      const int j = ops_first(Q) + u;  // this wave's MFMA index inside the fragment
      v8i bv;
      if constexpr (W == kFmtFp4) {
        // lane group g: k 32g .. 32g+31 of operand u (16 bytes)
        const v4i lo = *reinterpret_cast<const v4i*>(st + r * kBand + (((4 * u + g) ^ sw) << 4));
        bv = v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
      } else if constexpr (W == kFmtFp8) {
        // lane group g: k 16g .. 16g+15 and 64+16g .. 64+16g+15
        const v4i lo = *reinterpret_cast<const v4i*>(st + r * kBand + ((g ^ sw) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(st + r * kBand + (((4 + g) ^ sw) << 4));
        bv = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else if constexpr (LINE) {
        // lane group g: k 32g .. 32g+31, the 24 bytes at 96 j + 24 g of this
        // wave's band of the row, as three 8-byte pieces; a piece before
        // byte 128 Q lies in the previous stage (at most one stage back: an
        // operand is 96 bytes)
        int w6[6];
#pragma unroll
        for (int i = 0; i < 3; i++) {
          const int p = 96 * j + 24 * g + 8 * i - 128 * Q;  // -128 < p < 128
          const int back = p < 0 ? 1 : 0;
          const int o = p + 128 * back;
          const uint8_t* sb_ = t.wsm + ((f * NQ + Q - back) & (D - 1)) * STAGE;
          const v2i c = *reinterpret_cast<const v2i*>(sb_ + r * kBand + (((o >> 4) ^ sw) << 4) + (o & 8));
          w6[2 * i] = c[0];
          w6[2 * i + 1] = c[1];
        }
        bv = v8i{w6[0], w6[1], w6[2], w6[3], w6[4], w6[5], 0, 0};
      } else if constexpr (is_fp6(W)) {
        // lane group g: k 32g .. 32g+31, the 24 bytes at 24g of the row's
        // operand = pieces 2g and 2g + 1 (12 bytes each, in swizzled
        // 16-byte slots)
        const v4i lo = *reinterpret_cast<const v4i*>(st + r * kBand + (((2 * g) ^ sw) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(st + r * kBand + (((2 * g + 1) ^ sw) << 4));
        bv = v8i{lo[0], lo[1], lo[2], hi[0], hi[1], hi[2], 0, 0};
      } else if constexpr (W == kElemInt4) {
        const uint8_t* row = st + r * kBand;
        // the fp8 operand's k ranges, 8 bytes of INT4 codes each (bytes 8g
        // and 32 + 8g of operand u), remapped to E4M3 codes
        const v2i lo = *reinterpret_cast<const v2i*>(row + (((4 * u + (g >> 1)) ^ sw) << 4) + 8 * (g & 1));
        const v2i hi = *reinterpret_cast<const v2i*>(row + (((4 * u + 2 + (g >> 1)) ^ sw) << 4) + 8 * (g & 1));
        uint32_t e[8];
        int4x8_to_e4m3((uint32_t)lo[0], e[0], e[1]);
        int4x8_to_e4m3((uint32_t)lo[1], e[2], e[3]);
        int4x8_to_e4m3((uint32_t)hi[0], e[4], e[5]);
        int4x8_to_e4m3((uint32_t)hi[1], e[6], e[7]);
        bv = v8i{(int)e[0], (int)e[1], (int)e[2], (int)e[3], (int)e[4], (int)e[5], (int)e[6], (int)e[7]};
      } else {
        // the fp4 operand's k range, 8 bytes of INT2 codes (byte 8g of
        // operand u), remapped to E2M1 codes
        const uint8_t* row = st + r * kBand;
        const v2i c = *reinterpret_cast<const v2i*>(row + (((2 * u + (g >> 1)) ^ sw) << 4) + 8 * (g & 1));
        uint32_t e[4];
        int2x16_to_e2m1((uint32_t)c[0], e[0], e[1]);
        int2x16_to_e2m1((uint32_t)c[1], e[2], e[3]);
        bv = v8i{(int)e[0], (int)e[1], (int)e[2], (int)e[3], 0, 0, 0, 0};
      }
      const int sb = sc[r * SBW + 4 * j + g];
#pragma unroll
      for (int mb = 0; mb < MB; mb++)
        t.acc[mb][LINE ? 0 : u] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            bv, t.av[mb][j], t.acc[mb][LINE ? 0 : u], kBFmt, kFmtFp8, 0, sb, 0,
            (int)__builtin_amdgcn_ubfe(t.sa[mb][j], 8 * g, 8));
    }
  }

  template <bool FIRST, int... Q>
  static __device__ __forceinline__ void fragment(State& t, int f, std::integer_sequence<int, Q...>) {
    (stage<Q, FIRST>(t, f), ...);
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      v4f p = t.acc[mb][0];
#pragma unroll
      for (int u = 1; u < MPS; u++) p += t.acc[mb][u];
      reinterpret_cast<v4f*>(t.smem + OFF_PART + (PAIRED ? (f & 3) : (f & 1)) * SZ_PSLOT)[(mb * kDecWaves + t.wave) * 64 +
                                                                                        t.lane] = p;
#pragma unroll
      for (int u = 0; u < MPS; u++) t.acc[mb][u] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    // every wave's partial of fragment f is in LDS after the barrier; the
    // slot is written again NPSLOT fragments later, after a later barrier,
    // which the reducing wave reaches only once it has read it
    if constexpr (PAIRED) {
      // barrier after every odd fragment and after the last one; one row
      // block per fragment, reduced by wave ff % 8 as its (ff / 8)-th
      if ((f & 1) == 1 || f == t.nf - 1) {
        wg_barrier();
#pragma unroll
        for (int k = 0; k < 2; k++) {
          const int ff = f - 1 + k;
          if ((k == 1 || (f & 1) == 1) && t.wave == ff % kDecWaves) {
            const v4f c = reduce(t.smem, ff & 3, 0, t.lane);
            const int j = ff / kDecWaves;
            if (j < kHeld) {
#pragma unroll
              for (int i = 0; i < kHeld; i++)
                if (i == j) t.held[i] = c;
            } else {
              store_c(*t.a, t.f_begin + ff, 0, c, t.g, t.r);
            }
          }
        }
      }
      return;
    }
    wg_barrier();
    // the MB row blocks of the fragment are reduced by MB different waves:
    // block u = MB f + mb by wave u % 8, as its (u / 8)-th
#pragma unroll
    for (int mb = 0; mb < MB; mb++) {
      const int u = f * MB + mb;
      if (t.wave == u % kDecWaves) {
        const v4f c = reduce(t.smem, f & 1, mb, t.lane);
        const int j = u / kDecWaves;
        if (j < kHeld) {
#pragma unroll
          for (int i = 0; i < kHeld; i++)
            if (i == j) t.held[i] = c;
        } else {
          store_c(*t.a, t.f_begin + f, mb, c, t.g, t.r);  // past the held ones: correct, with stricter waits
        }
      }
    }
  }

  static __device__ __forceinline__ void run(const DecArgs& a, uint8_t* smem) {
    State t;
    t.a = &a;
    t.smem = smem;
    const int tid = threadIdx.x;
    t.lane = tid & 63;
    t.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    t.wsm = smem + t.wave * SZ_WAVE;
    t.kb = band_start(t.wave);
    t.g = t.lane >> 4;
    t.r = t.lane & 15;
    // balanced contiguous split of the fragments over the workgroups (each
    // has at least one: the grid is at most the fragment count)
    t.f_begin = (int)((int64_t)a.nfrags * blockIdx.x / gridDim.x);
    t.nf = (int)((int64_t)a.nfrags * (blockIdx.x + 1) / gridDim.x) - t.f_begin;
    if constexpr (is_fp6(W))
      t.rb = (uint32_t)((int64_t)a.ldk * OPB / 128);
    else
      t.rb = (uint32_t)(a.ldk / (128 / OPB));
    t.nb = (uint32_t)(a.ldk >> 5);
    // copy lane l: row l >> 3 (+8), physical chunk l & 7 holding logical chunk
    // (l & 7) ^ ((row >> 1) & 7)
    t.brow = t.lane >> 3;
#pragma unroll
    for (int h = 0; h < 2; h++)
      t.bch[h] = (uint32_t)(((t.lane & 7) ^ (((t.brow + 8 * h) >> 1) & 7)) * CPB);
    // scale copy i, lane l: entry e = 64 i + l is row e / LPR, dword e % LPR
    // (entries past row 15 repeat row 15 into the slot's unused tail)
#pragma unroll
    for (int i = 0; i < NSI; i++) {
      const int e = 64 * i + t.lane;
      t.srow[i] = min(e / LPR, 15);
      t.scol[i] = (uint32_t)(4 * (e % LPR));
    }

    prologue(t, std::make_integer_sequence<int, AHEAD>{});
#pragma unroll
    for (int mb = 0; mb < MB; mb++)
#pragma unroll
      for (int u = 0; u < MPS; u++) t.acc[mb][u] = v4f{0.f, 0.f, 0.f, 0.f};

    // the first fragment (exact wait counts while A is arriving), then the rest
    fragment<true>(t, 0, std::make_integer_sequence<int, NQ>{});
    for (int f = 1; f < t.nf; f++) fragment<false>(t, f, std::make_integer_sequence<int, NQ>{});
#pragma unroll
    for (int i = 0; i < kHeld; i++) {
      const int u = t.wave + kDecWaves * i;
      if (u / MB < t.nf) store_c(a, t.f_begin + u / MB, u % MB, t.held[i], t.g, t.r);
    }
    wait_vm<0>();  // no copy into LDS may still be in flight when the workgroup ends
  }
};

// the kernel's layout (the same for both wave kinds of an uneven split)
template <int W, int KW, int MB, int D>
using DecLayout = Decode<W, KW, MB, D, split_k(W, KW) ? 1 : 0>;

template <int W, int KW, int MB, int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512))) void decode_kernel(DecArgs a) {
  static_assert(DecLayout<W, KW, MB, D>::FITS, "fits the 160 KiB LDS of a gfx950 CU");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[DecLayout<W, KW, MB, D>::LDS];
  if constexpr (split_k(W, KW)) {
    static_assert(Decode<W, KW, MB, D, 1>::LDS == Decode<W, KW, MB, D, -1>::LDS, "one layout");
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
      Decode<W, KW, MB, D, 1>::run(a, smem);
    else
      Decode<W, KW, MB, D, -1>::run(a, smem);
  } else {
    Decode<W, KW, MB, D, 0>::run(a, smem);
  }
}

template <int W, int KW, int MB, int D = kDecStages>
hipError_t launch_dec(const DecArgs& a, int cus, hipStream_t stream) {
  const int grid = a.nfrags < cus ? a.nfrags : cus;
  hipLaunchKernelGGL((decode_kernel<W, KW, MB, D>), dim3(grid), dim3(kDecWaves * 64), 0, stream, a);
  return hipGetLastError();
}

// Row blocks of 16 activations per launch: the A operands of all blocks must
// fit 128 registers per lane (MB KW <= 16).
constexpr int max_blocks(int kw) { return kw <= 4 ? 4 : kw <= 8 ? 2 : 1; }

template <int W, int KW>
hipError_t launch_dec_m(const DecArgs& a, int cus, hipStream_t stream) {
  if (a.M <= 16 || max_blocks(KW) == 1) {
    // few weight fragments per CU: the ring covers a whole fragment
    if constexpr (DecLayout<W, KW, 1, kDecStagesDeep>::FITS) {
      if (a.nfrags <= kDeepMaxFrags * cus) return launch_dec<W, KW, 1, kDecStagesDeep>(a, cus, stream);
    }
    return launch_dec<W, KW, 1>(a, cus, stream);
  }
  if (W == kElemInt2 || a.M <= 32 || max_blocks(KW) == 2)  // INT2: at most 2 blocks (decode_ok)
    return launch_dec<W, KW, (max_blocks(KW) >= 2 ? 2 : 1)>(a, cus, stream);
  if constexpr (W != kElemInt2) return launch_dec<W, KW, max_blocks(KW)>(a, cus, stream);
  return hipErrorInvalidValue;
}

// Largest K / 1024: with fp8 weights (one MFMA per stage) the per-stage
// state of 14 or 16 MFMAs per wave no longer fits beside the A operands, and
// with INT4 weights the remapped operands of 16 MFMAs per wave (the compiler
// spills above 14).
constexpr int max_kw(int w) { return (w == kFmtFp8 || is_fp6(w)) ? 12 : w == kElemInt4 ? 14 : 16; }
// K / 1024 the kernel takes for a weight format: INT2 stages hold four MFMA
// operands, so every wave's band must be whole stages without a split
constexpr bool kw_ok(int w, int kw) { return kw >= 2 && kw <= max_kw(w) && (w != kElemInt2 || kw % 4 == 0); }

template <int W, int KW>
hipError_t launch_dec_kw(const DecArgs& a, int cus, hipStream_t stream) {
  if constexpr (!kw_ok(W, KW)) {
    return hipErrorInvalidValue;  // excluded by decode_ok
  } else {
    return launch_dec_m<W, KW>(a, cus, stream);
  }
}

template <int W, int... KW>
hipError_t launch_dec_k(const DecArgs& a, int cus, hipStream_t stream, std::integer_sequence<int, KW...>) {
  hipError_t err = hipErrorInvalidValue;  // K / 1024 outside 2 .. 16: excluded by decode_ok
  ((a.K == 1024 * (KW + 2) ? (err = launch_dec_kw<W, KW + 2>(a, cus, stream), 0) : 0), ...);
  return err;
}

// weight format of a (validated) format pair taken by the decode kernel
int weight_format(int fmt) {
  return fmt == 1 ? kFmtFp4 : fmt == 6 ? kElemInt4 : fmt == 7 ? kElemInt2 : fmt == 8 ? kFmtFp6 : fmt == 9 ? kFmtBf6
                                                                                                     : kFmtFp8;
}

// Rows of A one launch covers: 64 for K <= 4096, 32 for K <= 8192, 16
// above (the A operands of all row blocks fill the registers).  More rows
// take more launches, each streaming B once (16 x 28672 x 8192 fp8 x fp4,
// 33 .. 64 rows: 2 x 26-29 us, against 110-128 us for the split-K kernel).
int64_t rows_per_launch(int64_t K) { return 16 * max_blocks((int)(K / 1024)); }

// Longest K taken (in chunks above the per-launch range).
constexpr int64_t kDecMaxK = 131072;

// K / 1024 of chunk i of P: as equal as whole multiples of 1024 allow
int chunk_kw(int kw, int P, int i) { return kw / P + (i < kw % P ? 1 : 0); }

}  // namespace
bool decode_ok(int64_t M, int64_t K, int fmt, const uint8_t* SA, const uint8_t* SB, const Epi& e) {
  if (!(M <= 64 && (fmt == 0 || fmt == 1 || fmt == 6 || fmt == 7 || fmt == 8 || fmt == 9) && (K % 1024) == 0 &&
        K >= 2048 &&
        (((uintptr_t)SA | (uintptr_t)SB) & 3) == 0))
    return false;
  const int w = weight_format(fmt);
  // INT2: every chunk a multiple of 4096, and at most two blocks of 16 rows
  // (four blocks of A operands beside four remapped weight operands per
  // stage do not fit the registers)
  if (w == kElemInt2 && ((K % 4096) != 0 || M > 32)) return false;
  // above one launch's K range the running sum is kept in C between chunks,
  // which needs fp32 output
  return K <= 1024 * max_kw(w) || (e.out == kOutF32 && K <= kDecMaxK);
}

hipError_t launch_mx_decode(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                            int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream, int64_t kn) {
  if (kn < 0) kn = K;
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (cus <= 0) cus = 1;
  const int kw = (int)(kn / 1024);
  int P = 1;                               // K chunks
  int64_t step = rows_per_launch(kn);      // rows per launch
  if (e.out == kOutF32) {
    // fp32 C: one launch per K chunk covers all M rows, so that B streams
    // once; the chunks are the fewest whose A operands fit beside M / 16 row
    // blocks.  The first chunk writes C, each later one adds its partial sum,
    // and only the last applies bias and activation; the order is fixed, so
    // the result is deterministic.
    const int blocks = (int)((M + 15) / 16);
    const int limit = blocks <= 1 ? max_kw(weight_format(fmt)) : blocks <= 2 ? 8 : 4;  // max_blocks(KW) >= the blocks
    P = (kw + limit - 1) / limit;
    // INT2 chunks must stay multiples of 4096: the fewest such chunks
    if (weight_format(fmt) == kElemInt2) P = (kw / 4 + limit / 4 - 1) / (limit / 4);
    step = 64;
  }
  // (16-bit C: each launch takes all of K, which decode_ok keeps in range,
  // and launches of fewer rows stream B again)
  const int w = weight_format(fmt);
  const int64_t opb = op_bytes(w);  // weight bytes per 128 K elements
  for (int64_t m0 = 0; m0 < M && err == hipSuccess; m0 += step) {
    int64_t k0 = 0;
    for (int c = 0; c < P && err == hipSuccess; c++) {
      const int64_t kc = w == kElemInt2 ? 4096 * (int64_t)chunk_kw(kw / 4, P, c) : 1024 * (int64_t)chunk_kw(kw, P, c);
      DecArgs a{};
      a.A = (const uint8_t*)A + m0 * K + k0;  // E4M3 activations: one byte per element
      a.SA = SA + m0 * (K / 32) + k0 / 32;
      a.B = (const uint8_t*)B + k0 / 128 * opb;
      a.SB = SB + k0 / 32;
      a.e = c == P - 1 ? e : Epi{e.C, nullptr, kOutF32, kActNone};
      a.e.C = (uint8_t*)e.C + m0 * N * epi_elem_bytes(e.out);
      a.M = (int)(M - m0 < step ? M - m0 : step);
      a.N = (int)N;
      a.K = (int)kc;
      a.ldk = (int)K;
      a.accum = c > 0;
      a.nfrags = (int)((N + 15) / 16);
      const auto kws = std::make_integer_sequence<int, 15>{};  // K / 1024 = 2 .. 16
      err = w == kFmtFp4     ? launch_dec_k<kFmtFp4>(a, cus, stream, kws)
            : w == kElemInt4 ? launch_dec_k<kElemInt4>(a, cus, stream, kws)
            : w == kElemInt2 ? launch_dec_k<kElemInt2>(a, cus, stream, kws)
            : w == kFmtFp6   ? launch_dec_k<kFmtFp6>(a, cus, stream, kws)
            : w == kFmtBf6   ? launch_dec_k<kFmtBf6>(a, cus, stream, kws)
                             : launch_dec_k<kFmtFp8>(a, cus, stream, kws);
      k0 += kc;
    }
  }
  return err;
}

}  // namespace mxg
