// Row-wise kernels for gfx950: LayerNorm (pre-norm and final), fused QK
// normalisation + rotary embedding with the V transpose the attention kernel
// reads, and the element conversions used when weights are copied in.
//
// Method: "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
// section "How audio and speakers reach the language model" names QK
// normalisation and rotary position embeddings; the only norm the page names
// is LayerNorm.  Readings: LayerNorm with biased variance and eps = 1e-5;
// QK-norm is a LayerNorm over each head's 128 dims (one gain/bias pair for q,
// one for k, shared by the heads) applied before the rotation; the rotation
// turns pairs (i, i + 64) by p * 10000^(-i/64) with p the position in the clip.
//
// All of these are HBM-bound: one wavefront per row (or per row and head),
// statistics in fp32 registers with wavefront shuffles, vector loads/stores.

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr float LN_EPS = 1e-5f;

// One wavefront normalises one 1280-wide fp32 row; lane owns 5 float4 chunks.
__device__ __forceinline__ void ln_row_1280(const float* __restrict__ xr,
                                            const float* __restrict__ g,
                                            const float* __restrict__ b, int lane,
                                            float4 (&y)[5]) {
  float4 v[5];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    v[i] = *reinterpret_cast<const float4*>(xr + (i * 64 + lane) * 4);
    s += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  }
  const float mean = wave_sum(s) * (1.0f / D);
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    v[i].x -= mean; v[i].y -= mean; v[i].z -= mean; v[i].w -= mean;
    q += (v[i].x * v[i].x + v[i].y * v[i].y) + (v[i].z * v[i].z + v[i].w * v[i].w);
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.0f / D) + LN_EPS);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int c = (i * 64 + lane) * 4;
    const float4 gg = *reinterpret_cast<const float4*>(g + c);
    const float4 bb = *reinterpret_cast<const float4*>(b + c);
    y[i].x = v[i].x * rstd * gg.x + bb.x;
    y[i].y = v[i].y * rstd * gg.y + bb.y;
    y[i].z = v[i].z * rstd * gg.z + bb.z;
    y[i].w = v[i].w * rstd * gg.w + bb.w;
  }
}

__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ g,
                                                        const float* __restrict__ b,
                                                        bf16_t* __restrict__ y, int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float4 o[5];
  ln_row_1280(x + r * D, g, b, lane, o);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int c = (i * 64 + lane) * 4;
    *reinterpret_cast<uint2*>(y + r * D + c) =
        make_uint2(pack_bf16x2(o[i].x, o[i].y), pack_bf16x2(o[i].z, o[i].w));
  }
}

__global__ __launch_bounds__(256) void final_norm_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ b,
                                                         const int32_t* __restrict__ cu, int batch,
                                                         int64_t p_max, bf16_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= (int64_t)batch * p_max) return;
  const int bi = (int)(r / p_max);
  const int64_t p = r - (int64_t)bi * p_max;
  bf16_t* dst = out + r * D;
  if (p >= (int64_t)(cu[bi + 1] - cu[bi])) {
#pragma unroll
    for (int i = 0; i < 5; ++i)
      *reinterpret_cast<uint2*>(dst + (i * 64 + lane) * 4) = make_uint2(0u, 0u);
    return;
  }
  float4 o[5];
  ln_row_1280(x + ((int64_t)cu[bi] + p) * D, g, b, lane, o);
#pragma unroll
  for (int i = 0; i < 5; ++i)
    *reinterpret_cast<uint2*>(dst + (i * 64 + lane) * 4) =
        make_uint2(pack_bf16x2(o[i].x, o[i].y), pack_bf16x2(o[i].z, o[i].w));
}

// Workgroup: one attention tile (up to 128 positions of one clip) x one head.
// Each wavefront normalises and rotates q and k of 32 of the rows (lane holds
// dims i and i + 64, exactly a rotation pair); the workgroup then writes v
// transposed through LDS so that every store is 8 consecutive keys of one dim.
// The clip's keys occupy columns [vt_base[b], vt_base[b] + roundup(P_b, 64))
// of vt; columns past P_b are written as zeros.
constexpr int QK_ROWS = 128;

__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    bf16_t* __restrict__ qkv, const int32_t* __restrict__ cu, const int32_t* __restrict__ vt_base,
    const int32_t* __restrict__ tile_seq, const int32_t* __restrict__ tile_p0,
    const float* __restrict__ qg, const float* __restrict__ qb, const float* __restrict__ kg,
    const float* __restrict__ kb, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, bf16_t* __restrict__ vt, int64_t ld_vt) {
  __shared__ bf16_t sv[QK_ROWS][DH + 8];
  const int h = blockIdx.y;
  const int seq = tile_seq[blockIdx.x];
  const int p0 = tile_p0[blockIdx.x];
  const int64_t s0 = cu[seq];
  const int len = cu[seq + 1] - cu[seq];
  const int span = min(QK_ROWS, ((len + 63) & ~63) - p0);   // rows incl. zero padding
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  const float gq0 = qg[lane], gq1 = qg[lane + 64], bq0 = qb[lane], bq1 = qb[lane + 64];
  const float gk0 = kg[lane], gk1 = kg[lane + 64], bk0 = kb[lane], bk1 = kb[lane + 64];

  for (int rr = wave; rr < QK_ROWS; rr += 4) {
    const int p = p0 + rr;
    if (p >= len) break;
    const int64_t r = s0 + p;
    const float c = rope_cos[(int64_t)p * (DH / 2) + lane];
    const float s = rope_sin[(int64_t)p * (DH / 2) + lane];
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      bf16_t* base = qkv + r * (3 * D) + which * D + h * DH;
      const float a0 = bf16_to_f32(base[lane]);
      const float a1 = bf16_to_f32(base[lane + 64]);
      const float mean = wave_sum(a0 + a1) * (1.0f / DH);
      const float d0 = a0 - mean, d1 = a1 - mean;
      const float rstd = rsqrtf(wave_sum(d0 * d0 + d1 * d1) * (1.0f / DH) + LN_EPS);
      const float y0 = d0 * rstd * (which ? gk0 : gq0) + (which ? bk0 : bq0);
      const float y1 = d1 * rstd * (which ? gk1 : gq1) + (which ? bk1 : bq1);
      base[lane] = f32_to_bf16(y0 * c - y1 * s);
      base[lane + 64] = f32_to_bf16(y1 * c + y0 * s);
    }
  }

  // v tile -> LDS (row-major; rows past the clip are zero), then transposed out.
  for (int c = threadIdx.x; c < QK_ROWS * DH / 8; c += 256) {
    const int rr = c / (DH / 8), kc = c % (DH / 8);
    const int p = p0 + rr;
    uint4 u = make_uint4(0, 0, 0, 0);
    if (p < len) u = *reinterpret_cast<const uint4*>(qkv + (s0 + p) * (3 * D) + 2 * D + h * DH + kc * 8);
    *reinterpret_cast<uint4*>(&sv[rr][kc * 8]) = u;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < DH * QK_ROWS / 8; c += 256) {
    const int d = c / (QK_ROWS / 8), rc = c % (QK_ROWS / 8);
    if (rc * 8 >= span) continue;
    uint32_t e[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      e[q] = (uint32_t)sv[rc * 8 + 2 * q][d] | ((uint32_t)sv[rc * 8 + 2 * q + 1][d] << 16);
    bf16_t* dst = vt + ((int64_t)h * DH + d) * ld_vt + vt_base[seq] + p0 + rc * 8;
    *reinterpret_cast<uint4*>(dst) = make_uint4(e[0], e[1], e[2], e[3]);
  }
}

__global__ void to_bf16_kernel(const void* __restrict__ src, int src_is_bf16,
                               bf16_t* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (src_is_bf16) dst[i] = reinterpret_cast<const bf16_t*>(src)[i];
  else dst[i] = f32_to_bf16(reinterpret_cast<const float*>(src)[i]);
}

__global__ void to_f32_kernel(const void* __restrict__ src, int src_is_bf16,
                              float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (src_is_bf16) dst[i] = bf16_to_f32(reinterpret_cast<const bf16_t*>(src)[i]);
  else dst[i] = reinterpret_cast<const float*>(src)[i];
}

}  // namespace

hipError_t launch_layernorm(const float* x, const float* g, const float* b, bf16_t* y,
                            int64_t rows, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  layernorm_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(x, g, b, y, rows);
  return hipGetLastError();
}

hipError_t launch_final_norm(const float* x, const float* g, const float* b, const int32_t* cu_seq,
                             int batch, int64_t p_max, bf16_t* out, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * p_max;
  if (rows == 0) return hipSuccess;
  final_norm_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(
      x, g, b, cu_seq, batch, p_max, out);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(bf16_t* qkv, const int32_t* cu_seq, const int32_t* vt_base,
                              const int32_t* tile_seq, const int32_t* tile_p0, int n_tiles,
                              const float* qg, const float* qb, const float* kg, const float* kb,
                              const float* rope_cos, const float* rope_sin, bf16_t* vt,
                              int64_t ld_vt, hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  qknorm_rope_kernel<<<dim3(n_tiles, H), dim3(256), 0, stream>>>(
      qkv, cu_seq, vt_base, tile_seq, tile_p0, qg, qb, kg, kb, rope_cos, rope_sin, vt, ld_vt);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const void* src, bool src_is_bf16, bf16_t* dst, int64_t n,
                          hipStream_t stream) {
  if (n == 0) return hipSuccess;
  to_bf16_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
      src, src_is_bf16 ? 1 : 0, dst, n);
  return hipGetLastError();
}

hipError_t launch_to_f32(const void* src, bool src_is_bf16, float* dst, int64_t n,
                         hipStream_t stream) {
  if (n == 0) return hipSuccess;
  to_f32_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(
      src, src_is_bf16 ? 1 : 0, dst, n);
  return hipGetLastError();
}

}  // namespace enc
