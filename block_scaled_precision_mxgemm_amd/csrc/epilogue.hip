// epilogue.hip - the GEMM output step as a kernel of its own:
// Y[m][n] = out(act(X[m][n] + bias[n])) for an fp32 M x N matrix X, with the
// same device arithmetic as the epilogue fused into the GEMM kernels
// (mxg_epilogue.h), so the decomposed path (GEMM with fp32 C, then this
// kernel) and the fused one give identical bits.  "Resumo Técnico: RIGEL",
// section "4. Oportunidades de Otimização", compares exactly these two paths.
//
// Work mapping: one lane per 4 consecutive columns of a row (16-byte loads
// and stores when N % 4 == 0), grid-stride over the rows' column quads.  The
// kernel is bound by HBM bandwidth: 4 bytes read and 4 or 2 written per
// element (plus the bias row, read from cache).
#include "mxg_device.h"
#include "mxg_internal.h"

namespace mxg {
namespace {

__global__ __launch_bounds__(256) void epilogue_kernel(const float* __restrict__ X, int64_t M, int64_t N, Epi e) {
  const int64_t nq = (N + 3) >> 2;  // column quads per row
  const int64_t total = M * nq;
  const bool vec_rows = (N & 3) == 0;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total; u += step) {
    const int64_t m = u / nq;
    const int n = (int)((u - m * nq) << 2);
    const float* row = X + m * N;
    const bool vec = vec_rows && n + 3 < N;
    v4f v = {0.f, 0.f, 0.f, 0.f};
    if (vec) {
      v = *reinterpret_cast<const v4f*>(row + n);
    } else {
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (n + i < N) v[i] = row[n + i];
    }
    epi_store4<false>(e, N, m, n, v, vec);
  }
}

}  // namespace

hipError_t launch_epilogue(const float* X, int64_t M, int64_t N, const Epi& e, hipStream_t stream) {
  const int64_t total = M * ((N + 3) >> 2);
  int64_t grid = (total + 255) / 256;
  if (grid > 256 * 16) grid = 256 * 16;
  hipLaunchKernelGGL(epilogue_kernel, dim3((unsigned)grid), dim3(256), 0, stream, X, M, N, e);
  return hipGetLastError();
}

}  // namespace mxg
