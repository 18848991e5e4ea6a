// gemm_skinny.hip - MX GEMM for decode shapes (M <= 64 rows of activations
// against a large weight matrix).  Such a product is bound by the bytes of
// B, which must stream from HBM exactly once; the weight plane is what
// quantization shrinks ("Metal tensors でカスタム機械学習オペレーションを
// 最適化する", section "主要内容": inference is memory-bandwidth bound and
// quantization cuts both the footprint and the traffic).
//
// Design (gfx950):
//   * no LDS staging of B: every lane loads its MFMA operand bytes straight
//     from global memory (16-byte loads) in the scaled-MFMA register layout,
//     so each B byte is read once and used once;
//   * a workgroup owns NF * 16 columns of C (rows of B); its W waves split
//     the K range W ways (split-K) and the partial sums are added in LDS
//     in a fixed order, so the result is deterministic and needs no atomics
//     and no zero-initialised output.  NF is the largest of 4 (2 for M > 32),
//     2, 1 that still gives every CU a workgroup, and W = 8 when NF is
//     below that maximum (16 x 8192 x 28672 fp8 x fp4: 55 against 88 us;
//     16 x 1024 x 11008: 13 against 30 us; 16 x 28672 x 5120 keeps NF = 4,
//     W = 4);
//   * each wave keeps two groups of U slices in flight (registers), loading
//     group j+1 while the MFMAs of group j run;
//   * the activation rows (<= 64, a few hundred KiB) are re-read from L2 by
//     every workgroup.
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

struct SkArgs {
  const uint8_t* A;
  const uint8_t* SA;
  const uint8_t* B;
  const uint8_t* SB;
  Epi e;             // output: C, bias, activation, element type
  int M, N, K;       // K: the k range of this launch (A, B and scales start at its first element)
  int64_t lda, ldb;  // row strides in bytes
  int64_t lds;       // row stride of the scale planes in bytes
  int accum;         // 1: fp32 C already holds the sum over the k before this range; add to it
  int nslices;       // ceil(K / 128)
};

// WF: weight format (kFmtFp8, kFmtFp4, kElemInt4, kElemInt2, kFmtFp6 or
// kFmtBf6; the integer codes are remapped in registers to E4M3 / E2M1 MFMA
// operands, the FP6 codes are MFMA operands as stored)
template <int MT, int NF, int WF, int U, int W>
struct Skinny {
  static constexpr bool FP6 = WF == kFmtFp6 || WF == kFmtBf6;
  // MFMA format of B
  static constexpr int BFMT = FP6 ? WF : (WF == kFmtFp8 || WF == kElemInt4) ? kFmtFp8 : kFmtFp4;
  struct Group {
    v8i a[U][MT];
    v8i b[U][NF];
    int sa[U][MT];
    int sb[U][NF];
  };

  // fp8 operand bytes of one lane: k = 16g..16g+15 and 64+16g..64+16g+15
  static __device__ __forceinline__ v8i load_fp8(const uint8_t* row, int k0, int g, int K) {
    v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
    if (k0 + 16 * g < K) lo = *reinterpret_cast<const v4i*>(row + k0 + 16 * g);
    if (k0 + 64 + 16 * g < K) hi = *reinterpret_cast<const v4i*>(row + k0 + 64 + 16 * g);
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // fp4 operand bytes of one lane: k = 32g..32g+31 (16 bytes)
  static __device__ __forceinline__ v8i load_fp4(const uint8_t* row, int k0, int g, int K) {
    v4i lo = {0, 0, 0, 0};
    if (k0 + 32 * g < K) lo = *reinterpret_cast<const v4i*>(row + (k0 >> 1) + 16 * g);
    return v8i{lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
  }
  // INT4 codes of the fp8 operand's k ranges (8 bytes each), remapped to E4M3
  static __device__ __forceinline__ v8i load_int4(const uint8_t* row, int k0, int g, int K) {
    v2i lo = {0, 0}, hi = {0, 0};
    if (k0 + 16 * g < K) lo = *reinterpret_cast<const v2i*>(row + (k0 >> 1) + 8 * g);
    if (k0 + 64 + 16 * g < K) hi = *reinterpret_cast<const v2i*>(row + (k0 >> 1) + 32 + 8 * g);
    uint32_t e[8];
    int4x8_to_e4m3((uint32_t)lo[0], e[0], e[1]);
    int4x8_to_e4m3((uint32_t)lo[1], e[2], e[3]);
    int4x8_to_e4m3((uint32_t)hi[0], e[4], e[5]);
    int4x8_to_e4m3((uint32_t)hi[1], e[6], e[7]);
    return v8i{(int)e[0], (int)e[1], (int)e[2], (int)e[3], (int)e[4], (int)e[5], (int)e[6], (int)e[7]};
  }
  // INT2 codes of the fp4 operand's k range (8 bytes), remapped to E2M1
  static __device__ __forceinline__ v8i load_int2(const uint8_t* row, int k0, int g, int K) {
    v2i c = {0, 0};
    if (k0 + 32 * g < K) c = *reinterpret_cast<const v2i*>(row + (k0 >> 2) + 8 * g);
    uint32_t e[4];
    int2x16_to_e2m1((uint32_t)c[0], e[0], e[1]);
    int2x16_to_e2m1((uint32_t)c[1], e[2], e[3]);
    return v8i{(int)e[0], (int)e[1], (int)e[2], (int)e[3], 0, 0, 0, 0};
  }
  // FP6 operand bytes of one lane: k = 32g .. 32g+31, 24 bytes (6 registers;
  // element i of the lane at bits 6i .. 6i+5, as the rows store them)
  static __device__ __forceinline__ v8i load_fp6(const uint8_t* row, int k0, int g, int K) {
    v2i a = {0, 0}, b = {0, 0}, c = {0, 0};
    const uint8_t* p = row + (k0 >> 2) * 3 + 24 * g;
    if (k0 + 32 * g < K) {
      a = *reinterpret_cast<const v2i*>(p);
      b = *reinterpret_cast<const v2i*>(p + 8);
      c = *reinterpret_cast<const v2i*>(p + 16);
    }
    return v8i{a[0], a[1], b[0], b[1], c[0], c[1], 0, 0};
  }
  static __device__ __forceinline__ int load_scale(const uint8_t* srow, int blk, int nb) {
    return (blk < nb) ? (int)srow[blk] : 127;
  }

  static __device__ __forceinline__ void load_group(const SkArgs& a, int n0, int s, int s_end, int g, int r,
                                                    Group& G) {
    const int nb = a.K >> 5;
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int sl = s + u;
      const bool live = sl < s_end;
      const int k0 = sl * 128;
#pragma unroll
      for (int j = 0; j < NF; j++) {
        const int n = min(n0 + j * 16 + r, a.N - 1);
        const uint8_t* brow = a.B + (int64_t)n * a.ldb;
        if (live) {
          if constexpr (FP6)
            G.b[u][j] = load_fp6(brow, k0, g, a.K);
          else
            G.b[u][j] = WF == kFmtFp4     ? load_fp4(brow, k0, g, a.K)
                        : WF == kElemInt4 ? load_int4(brow, k0, g, a.K)
                        : WF == kElemInt2 ? load_int2(brow, k0, g, a.K)
                                          : load_fp8(brow, k0, g, a.K);
          G.sb[u][j] = load_scale(a.SB + (int64_t)n * a.lds, sl * 4 + g, nb);
        } else {
          G.b[u][j] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          G.sb[u][j] = 127;
        }
      }
#pragma unroll
      for (int t = 0; t < MT; t++) {
        const int m = min(t * 16 + r, a.M - 1);
        const uint8_t* arow = a.A + (int64_t)m * a.lda;
        if (live) {
          G.a[u][t] = load_fp8(arow, k0, g, a.K);
          G.sa[u][t] = load_scale(a.SA + (int64_t)m * a.lds, sl * 4 + g, nb);
        } else {
          G.a[u][t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          G.sa[u][t] = 127;
        }
      }
    }
  }

  static __device__ __forceinline__ void compute(const Group& G, v4f (&acc)[MT][NF]) {
#pragma unroll
    for (int u = 0; u < U; u++)
#pragma unroll
      for (int t = 0; t < MT; t++)
#pragma unroll
        for (int j = 0; j < NF; j++)
          acc[t][j] = mfma_scaled_16x16x128<BFMT, kFmtFp8>(G.b[u][j], G.a[u][t], acc[t][j], G.sb[u][j],
                                                           G.sa[u][t]);
  }

  static __device__ __forceinline__ void run(const SkArgs& a) {
    __shared__ v4f red[W - 1][MT][NF][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const int n0 = blockIdx.x * NF * 16;
    // K split: wave w takes slices [s_begin, s_end)
    const int per = (a.nslices + W - 1) / W;
    const int s_begin = min(wave * per, a.nslices);
    const int s_end = min(s_begin + per, a.nslices);

    v4f acc[MT][NF];
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
      for (int j = 0; j < NF; j++) acc[t][j] = v4f{0.f, 0.f, 0.f, 0.f};

    Group cur, nxt;
    if (s_begin < s_end) load_group(a, n0, s_begin, s_end, g, r, cur);
    for (int s = s_begin; s < s_end; s += U) {
      if (s + U < s_end) load_group(a, n0, s + U, s_end, g, r, nxt);
      compute(cur, acc);
      cur = nxt;
    }

    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < MT; t++)
#pragma unroll
        for (int j = 0; j < NF; j++) red[wave - 1][t][j][lane] = acc[t][j];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < MT; t++) {
      const int m = t * 16 + r;
#pragma unroll
      for (int j = 0; j < NF; j++) {
        v4f v = acc[t][j];
#pragma unroll
        for (int w = 0; w < W - 1; w++) v += red[w][t][j][lane];
        if (m >= a.M) continue;
        const int n = n0 + j * 16 + 4 * g;
        const bool vec = (a.N & 3) == 0 && n + 3 < a.N;
        if (a.accum) {
          const float* prev = reinterpret_cast<const float*>(a.e.C) + (int64_t)m * a.N + n;
          if (vec) {
            v += *reinterpret_cast<const v4f*>(prev);
          } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
              if (n + i < a.N) v[i] += prev[i];
          }
        }
        epi_store4<false>(a.e, a.N, m, n, v, vec);
      }
    }
  }
};

template <int MT, int NF, int WF, int U, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(W * 64, W * 64))) void skinny_kernel(SkArgs a) {
  Skinny<MT, NF, WF, U, W>::run(a);
}

template <int MT, int NF, int WF, int U, int W = 4>
hipError_t launch_sk(const SkArgs& a, hipStream_t stream) {
  const int grid = (a.N + NF * 16 - 1) / (NF * 16);
  hipLaunchKernelGGL((skinny_kernel<MT, NF, WF, U, W>), dim3(grid), dim3(W * 64), 0, stream, a);
  return hipGetLastError();
}

// Column width (fragments per workgroup) and K split: the widest of NFMAX,
// 2, 1 fragments that still gives every CU a workgroup, with 8 waves
// splitting K when narrower than NFMAX.
template <int MT, int NFMAX, int WF>
hipError_t launch_by_n(const SkArgs& a, hipStream_t stream) {
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const int64_t frags = (a.N + 15) / 16;
  if (frags >= NFMAX * (int64_t)cus) return launch_sk<MT, NFMAX, WF, 2, 4>(a, stream);
  if (NFMAX > 2 && frags >= 2 * (int64_t)cus) return launch_sk<MT, (NFMAX > 2 ? 2 : 1), WF, 2, 8>(a, stream);
  return launch_sk<MT, 1, WF, 2, 8>(a, stream);
}

template <int WF>
hipError_t launch_by_m(const SkArgs& a, hipStream_t stream) {
  if (a.M <= 16) return launch_by_n<1, 4, WF>(a, stream);
  if (a.M <= 32) return launch_by_n<2, 4, WF>(a, stream);
  return launch_by_n<4, 2, WF>(a, stream);
}

}  // namespace

hipError_t launch_mx_skinny(const void* A, const uint8_t* SA, const void* B, const uint8_t* SB, const Epi& e,
                            int64_t M, int64_t N, int64_t K, int fmt, hipStream_t stream, int64_t k0, int64_t kn) {
  if (kn < 0) kn = K - k0;
  SkArgs a{};
  a.A = (const uint8_t*)A + k0;  // E4M3 activations: one byte per element
  a.SA = SA + k0 / 32;
  // weight bytes per 4 elements: 4 (E4M3), 2 (E2M1, INT4), 1 (INT2), 3 (FP6)
  const int64_t b4 = fmt == 0 ? 4 : fmt == 7 ? 1 : (fmt == 8 || fmt == 9) ? 3 : 2;
  a.B = (const uint8_t*)B + k0 / 4 * b4;
  a.SB = SB + k0 / 32;
  a.e = e;
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)kn;
  a.lda = K;
  a.ldb = K / 4 * b4;
  a.lds = K / 32;
  a.accum = k0 > 0;
  a.nslices = (int)((kn + 127) / 128);
  switch (fmt) {
    case 0: return launch_by_m<kFmtFp8>(a, stream);
    case 1: return launch_by_m<kFmtFp4>(a, stream);
    case 6: return launch_by_m<kElemInt4>(a, stream);
    case 8: return launch_by_m<kFmtFp6>(a, stream);
    case 9: return launch_by_m<kFmtBf6>(a, stream);
    default: return launch_by_m<kElemInt2>(a, stream);
  }
}

}  // namespace mxg
