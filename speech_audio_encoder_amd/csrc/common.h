// Shared device helpers for the gfx950 kernels: bf16 storage, MFMA operand
// vector types, wavefront reductions, and the launchers' internal interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace enc {

// Model constants of the encoder (width, heads, head width, FFN width,
// stacked input width, mel bands) and of the frontend (window, hop, transform).
constexpr int D = 1280;
constexpr int H = 10;
constexpr int DH = 128;
constexpr int FF = 5120;
constexpr int DIN = 1024;
constexpr int NMEL = 128;
constexpr int STACK = 8;
constexpr int WIN = 400;
constexpr int HOP = 160;
constexpr int NFFT = 512;
constexpr int NBIN = 257;
constexpr int64_t MAX_SAMPLES = 57600000;   // one hour at 16 kHz
constexpr int MAX_POS = 45000;              // positions of a one-hour clip

typedef uint16_t bf16_t;   // bfloat16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest, ties to even.  Inputs here are finite.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace enc
