// mfma_ceiling.hip - measurement helper: the matrix-core throughput the chip
// sustains on a given operand distribution, with no memory traffic.
//
// The large GEMM's compute phase issues 32 scaled MFMAs per wave (8 A x 4 B
// fragments of 16 rows, 128 K each); the chip's clock under that load depends
// on the operand bits (switching activity), so its published peak is not what
// random data can reach.  This kernel runs exactly that phase back to back on
// fragments loaded once from the caller's operand bytes (the benchmark passes
// the workload's own quantized codes and scales), two waves per SIMD like the
// GEMM, and nothing else: its rate is the ceiling a kernel feeding the
// matrix cores perfectly would meet on that data.  The benchmark reports it
// beside the published peak, in the manner of a measured roofline ("Resumo
// Técnico: RIGEL", section "Metodologia: O Harness RIGEL", throughput
// ceilings triangulated by measurement).
#include <string.h>

#include <utility>

#include "../../include/mxgemm.h"
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

template <int FA, int FB, int... I>
__device__ __forceinline__ void phase_scaled(v4f (&acc)[8][4], const v8i (&af)[8], const v8i (&bf)[4],
                                             const int (&sa)[2], int sb, std::integer_sequence<int, I...>) {
  (mfma_scaled_acc_pk<FB, FA, I / 8, (I % 8) & 3>(acc[I % 8][I / 8], bf[I / 8], af[I % 8], sb, sa[(I % 8) >> 2]),
   ...);
}

// One float per lane of every wave goes to out (the sum of its
// accumulators), so no MFMA can be removed as dead code.  With clocks set,
// wave 0 of every workgroup also records the shader-clock cycles
// (s_memtime) and the 100 MHz constant-clock ticks (s_memrealtime) that its
// MFMA loop took: their ratio is the shader clock under this load.
template <int KIND, int FA, int FB>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void ceiling_kernel(const uint8_t* ops, int64_t op_bytes, const uint8_t* scales, int64_t scale_bytes, int iters,
                    float* out, uint32_t* clocks) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 6);
  // fragment f of this wave: 32 bytes per lane at a position that differs
  // per wave, fragment and lane (wrapping inside the buffer)
  const int64_t chunks = op_bytes / 32;
  v8i af[8], bf[4];
#pragma unroll
  for (int f = 0; f < 12; f++) {
    const int64_t c = ((gw * 12 + f) * 64 + lane) % chunks;
    const v4i lo = *reinterpret_cast<const v4i*>(ops + c * 32);
    const v4i hi = *reinterpret_cast<const v4i*>(ops + c * 32 + 16);
    const v8i v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    if (f < 8)
      af[f] = v;
    else
      bf[f - 8] = v;
  }
  int sa[2] = {0, 0}, sb = 0;
  if (KIND == 0) {
    const int64_t words = scale_bytes / 4;
    sa[0] = reinterpret_cast<const int*>(scales)[(gw * 192 + lane) % words];
    sa[1] = reinterpret_cast<const int*>(scales)[(gw * 192 + 64 + lane) % words];
    sb = reinterpret_cast<const int*>(scales)[(gw * 192 + 128 + lane) % words];
  }
  v4f acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  mfma_fence_init(acc);
  // operands written by loads (and VALU moves) are ready, with the wait
  // states an MFMA needs after a VALU write, before the first MFMA
  asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 4"
               : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]), "+v"(af[4]), "+v"(af[5]), "+v"(af[6]),
                 "+v"(af[7]), "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]), "+v"(bf[3]), "+v"(sa[0]), "+v"(sa[1]), "+v"(sb)
               :
               : "memory");
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it++) {
    if constexpr (KIND == 0) {
      phase_scaled<FA, FB>(acc, af, bf, sa, sb, std::make_integer_sequence<int, 32>{});
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
  }
  mfma_drain(acc);
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (clocks != nullptr && threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = (uint32_t)(t1 - t0);
    clocks[2 * blockIdx.x + 1] = (uint32_t)(r1 - r0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) s += acc[i][j][0] + acc[i][j][1] + acc[i][j][2] + acc[i][j][3];
  out[gw * 64 + lane] = s;
}

template <int KIND, int FA, int FB>
hipError_t launch_ceiling(const uint8_t* ops, int64_t op_bytes, const uint8_t* scales, int64_t scale_bytes,
                          int iters, int workgroups, float* out, uint32_t* clocks, hipStream_t st) {
  hipLaunchKernelGGL((ceiling_kernel<KIND, FA, FB>), dim3((unsigned)workgroups), dim3(512), 0, st, ops, op_bytes,
                     scales, scale_bytes, iters, out, clocks);
  return hipGetLastError();
}

}  // namespace
}  // namespace mxg

extern "C" int mxgemm_mfma_ceiling(const void* ops, int64_t op_bytes, const uint8_t* scales, int64_t scale_bytes,
                                   int kind, int64_t iters, int workgroups, float* out, uint32_t* clocks,
                                   void* stream) {
  using namespace mxg;
  if (!ops || !out || op_bytes < 32 || iters < 1 || iters > (1 << 30) || workgroups < 1 || workgroups > (1 << 20))
    return MXG_EINVAL;
  if (kind != MXG_CEIL_FP16 && (kind < MXG_FMT_FP8_FP8 || kind > MXG_FMT_BF8_FP8)) return MXG_EINVAL;
  if (kind != MXG_CEIL_FP16 && (!scales || scale_bytes < 4)) return MXG_EINVAL;
  if (((uintptr_t)ops & 15) || ((uintptr_t)out & 15) || (scales && ((uintptr_t)scales & 3)) ||
      ((uintptr_t)clocks & 3))
    return MXG_EALIGN;
  int dev = 0;
  hipDeviceProp_t p;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess) return MXG_EHIP;
  if (strncmp(p.gcnArchName, "gfx950", 6) != 0) return MXG_EUNSUPPORTED;
  const hipStream_t st = (hipStream_t)stream;
  const uint8_t* o = (const uint8_t*)ops;
  const int it = (int)iters;
  hipError_t e;
  switch (kind) {
    case MXG_FMT_FP8_FP8: e = launch_ceiling<0, kFmtFp8, kFmtFp8>(o, op_bytes, scales, scale_bytes, it, workgroups, out, clocks, st); break;
    case MXG_FMT_FP8_FP4: e = launch_ceiling<0, kFmtFp8, kFmtFp4>(o, op_bytes, scales, scale_bytes, it, workgroups, out, clocks, st); break;
    case MXG_FMT_FP4_FP4: e = launch_ceiling<0, kFmtFp4, kFmtFp4>(o, op_bytes, scales, scale_bytes, it, workgroups, out, clocks, st); break;
    case MXG_FMT_BF8_BF8: e = launch_ceiling<0, kFmtBf8, kFmtBf8>(o, op_bytes, scales, scale_bytes, it, workgroups, out, clocks, st); break;
    case MXG_FMT_FP8_BF8: e = launch_ceiling<0, kFmtFp8, kFmtBf8>(o, op_bytes, scales, scale_bytes, it, workgroups, out, clocks, st); break;
    case MXG_FMT_BF8_FP8: e = launch_ceiling<0, kFmtBf8, kFmtFp8>(o, op_bytes, scales, scale_bytes, it, workgroups, out, clocks, st); break;
    default: e = launch_ceiling<1, kFmtFp8, kFmtFp8>(o, op_bytes, scales, scale_bytes, it, workgroups, out, clocks, st); break;
  }
  return e == hipSuccess ? MXG_OK : MXG_EHIP;
}
