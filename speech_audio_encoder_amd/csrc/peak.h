// Device probes (peak.hip): a register-only loop of dense bf16 MFMAs and a
// device copy, which measure what the device sustains.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace enc {

// Dense bf16 flops of one launch of launch_mfma_loop(out, grid, iters).
int64_t mfma_loop_flops(int grid, int iters);
// grid workgroups of four wavefronts, each issuing iters x 8 MFMAs
// (v_mfma_f32_32x32x16_bf16); out receives grid x 256 floats.
hipError_t launch_mfma_loop(float* out, int grid, int iters, hipStream_t stream);
// dst = src over `bytes` bytes (bytes % 16 == 0), 16 bytes per lane.
hipError_t launch_copy16(void* dst, const void* src, size_t bytes, hipStream_t stream);

}  // namespace enc
