// Probes of what the device sustains, the context for every roofline
// fraction: back-to-back dense bf16 MFMAs with operands in registers (no
// memory traffic), and a plain device-to-device copy.  The published MI355X
// figures (2.5 PFLOP/s dense bf16 at 2.4 GHz, 8 TB/s HBM) assume the peak
// clock and ideal DRAM efficiency; these kernels measure what one launch of
// each actually reaches on the device at hand.

#include "common.h"
#include "peak.h"

namespace enc {

namespace {

constexpr int MFMA_CHAINS = 8;   // independent accumulators per wavefront

// Every wavefront issues iters x MFMA_CHAINS v_mfma_f32_32x32x16_bf16 on
// register operands; eight independent accumulators keep the matrix core fed
// without waiting on a result.  The sums are stored so the work stays live.
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
  }
  f32x16 acc[MFMA_CHAINS];
#pragma unroll
  for (int k = 0; k < MFMA_CHAINS; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < MFMA_CHAINS; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < MFMA_CHAINS; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// dst[i] = src[i] over n 16-byte chunks, four per thread, each load and
// store instruction covering 1 KB contiguous per wavefront.
__global__ __launch_bounds__(256) void copy16_kernel(uint4* __restrict__ dst,
                                                     const uint4* __restrict__ src, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  uint4 v[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t i = base + t * 256;
    if (i < n) v[t] = src[i];
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t i = base + t * 256;
    if (i < n) dst[i] = v[t];
  }
}

}  // namespace

int64_t mfma_loop_flops(int grid, int iters) {
  return (int64_t)grid * 4 * iters * MFMA_CHAINS * (2LL * 32 * 32 * 16);
}

hipError_t launch_mfma_loop(float* out, int grid, int iters, hipStream_t stream) {
  if (grid < 1 || iters < 1) return hipErrorInvalidValue;
  mfma_loop_kernel<<<dim3(grid), dim3(256), 0, stream>>>(out, iters);
  return hipGetLastError();
}

hipError_t launch_copy16(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  copy16_kernel<<<dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, stream>>>(
      reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), n);
  return hipGetLastError();
}

}  // namespace enc
