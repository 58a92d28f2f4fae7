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
constexpr int NSPK = 8;                     // speaker slots of the activity input
// Scale applied to k after QK-norm and rotation: log2(e) / sqrt(head dim),
// so that q . k is the softmax exponent in base 2.
constexpr float K_SCORE_SCALE = 0.12751743082459868f;

typedef uint16_t bf16_t;   // bfloat16 bits in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// Round to nearest, ties to even: gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_v v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// E4M3 (OCP FP8) codes of four values: saturated at +-448, then rounded to
// nearest even by v_cvt_pk_fp8_f32; byte i of the result holds value i.
constexpr float E4M3_MAX = 448.0f;
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -E4M3_MAX), E4M3_MAX);
  b = fminf(fmaxf(b, -E4M3_MAX), E4M3_MAX);
  c = fminf(fmaxf(c, -E4M3_MAX), E4M3_MAX);
  d = fminf(fmaxf(d, -E4M3_MAX), E4M3_MAX);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)lo, true);
}

// Wavefront reductions (every lane of the wavefront active; every lane gets
// the result).  Inside each row of 16 lanes, DPP moves (quad permutations
// [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors) leave the row's
// total in all of its lanes without touching LDS; the four row totals are then
// read from lanes 0, 16, 32 and 48.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}

template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_move<0x141>(v));   // row_half_mirror
  v = op(v, dpp_move<0x140>(v));   // row_mirror
  auto lane = [&](int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  };
  return op(op(lane(0), lane(16)), op(lane(32), lane(48)));
}

// Sum over each aligned group of 8 lanes, in all 8 (the quad permutations
// and the half-row mirror of the reduction above).
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp_move<0xB1>(v);
  v += dpp_move<0x4E>(v);
  return v + dpp_move<0x141>(v);
}

__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

}  // namespace enc
