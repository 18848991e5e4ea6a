// lds_poison.hip - test helper (not part of the library): fills the LDS of
// every compute unit with one 32-bit pattern, so that a kernel launched
// next which reads an LDS location before writing it sees the pattern
// instead of whatever an earlier kernel left there.  With 0xFFFFFFFF the
// stale bytes decode as NaN E4M3 codes, NaN UE8M0 scales, -6 E2M1 nibbles
// and NaN fp32 partial sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
constexpr int kWords = 160 * 1024 / 4;  // the whole 160 KiB of a gfx950 CU

__global__ __launch_bounds__(1024) void poison_lds_kernel(uint32_t word) {
  __shared__ uint32_t lds[kWords];
  volatile uint32_t* p = lds;  // volatile: the stores are the point
  for (int i = threadIdx.x; i < kWords; i += blockDim.x) p[i] = word;
  __syncthreads();
}
}  // namespace

// Enqueues enough workgroups (each holding all of a CU's LDS) to visit every
// CU several times.  Returns 0, or the HIP error code of the launch.
extern "C" int lds_poison(uint32_t word, int workgroups, void* stream) {
  hipLaunchKernelGGL(poison_lds_kernel, dim3((unsigned)workgroups), dim3(1024), 0, (hipStream_t)stream, word);
  return (int)hipGetLastError();
}
