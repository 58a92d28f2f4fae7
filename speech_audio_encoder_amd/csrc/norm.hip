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
// The wavefronts normalise and rotate q and k of the tile's rows, then each
// thread transposes an 8 x 8 block of v in registers so that every store is 8
// consecutive keys of one dim.
// The clip's keys occupy columns [vt_base[b], vt_base[b] + roundup(P_b, 64))
// of vt; columns past P_b are written as zeros.
constexpr int QK_ROWS = 128;

__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    bf16_t* __restrict__ qkv, const int32_t* __restrict__ cu, const int32_t* __restrict__ vt_base,
    const int32_t* __restrict__ tile_seq, const int32_t* __restrict__ tile_p0,
    const float* __restrict__ qg, const float* __restrict__ qb, const float* __restrict__ kg,
    const float* __restrict__ kb, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, bf16_t* __restrict__ vt, int64_t ld_vt) {
  const int h = blockIdx.y;
  const int seq = tile_seq[blockIdx.x];
  const int p0 = tile_p0[blockIdx.x];
  const int64_t s0 = cu[seq];
  const int len = cu[seq + 1] - cu[seq];
  const int span = min(QK_ROWS, ((len + 63) & ~63) - p0);   // rows incl. zero padding
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // q and k: 16 lanes per (row, head); lane j of a group holds dims 4j..4j+3
  // and 64+4j..64+4j+3, i.e. four whole rotation pairs, so the rotation is
  // local and every access is an 8-byte vector.  A wavefront does 4 rows at a
  // time; the statistics reduce over the 16 lanes of the group.
  const int sub = lane & 15;
  const int grp = lane >> 4;
  const int d0 = sub * 4;
  const float4 gq0 = *reinterpret_cast<const float4*>(qg + d0);
  const float4 gq1 = *reinterpret_cast<const float4*>(qg + 64 + d0);
  const float4 bq0 = *reinterpret_cast<const float4*>(qb + d0);
  const float4 bq1 = *reinterpret_cast<const float4*>(qb + 64 + d0);
  const float4 gk0 = *reinterpret_cast<const float4*>(kg + d0);
  const float4 gk1 = *reinterpret_cast<const float4*>(kg + 64 + d0);
  const float4 bk0 = *reinterpret_cast<const float4*>(kb + d0);
  const float4 bk1 = *reinterpret_cast<const float4*>(kb + 64 + d0);

  for (int rr = wave * 4 + grp; rr < QK_ROWS; rr += 16) {
    const int p = p0 + rr;
    if (p >= len) continue;
    const int64_t r = s0 + p;
    const float4 c = *reinterpret_cast<const float4*>(rope_cos + (int64_t)p * (DH / 2) + d0);
    const float4 sn = *reinterpret_cast<const float4*>(rope_sin + (int64_t)p * (DH / 2) + d0);
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      bf16_t* base = qkv + r * (3 * D) + which * D + h * DH;
      const uint2 ulo = *reinterpret_cast<const uint2*>(base + d0);
      const uint2 uhi = *reinterpret_cast<const uint2*>(base + 64 + d0);
      float a[4] = {bf16_to_f32((bf16_t)(ulo.x & 0xFFFF)), bf16_to_f32((bf16_t)(ulo.x >> 16)),
                    bf16_to_f32((bf16_t)(ulo.y & 0xFFFF)), bf16_to_f32((bf16_t)(ulo.y >> 16))};
      float b[4] = {bf16_to_f32((bf16_t)(uhi.x & 0xFFFF)), bf16_to_f32((bf16_t)(uhi.x >> 16)),
                    bf16_to_f32((bf16_t)(uhi.y & 0xFFFF)), bf16_to_f32((bf16_t)(uhi.y >> 16))};
      float sum = (a[0] + a[1]) + (a[2] + a[3]) + (b[0] + b[1]) + (b[2] + b[3]);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
      const float mean = sum * (1.0f / DH);
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] -= mean;
        b[e] -= mean;
        sq += a[e] * a[e] + b[e] * b[e];
      }
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) sq += __shfl_xor(sq, o, 64);
      const float rstd = rsqrtf(sq * (1.0f / DH) + LN_EPS);
      const float4 g0 = which ? gk0 : gq0, g1 = which ? gk1 : gq1;
      const float4 e0 = which ? bk0 : bq0, e1 = which ? bk1 : bq1;
      const float ga[4] = {g0.x, g0.y, g0.z, g0.w}, gb[4] = {g1.x, g1.y, g1.z, g1.w};
      const float ea[4] = {e0.x, e0.y, e0.z, e0.w}, eb[4] = {e1.x, e1.y, e1.z, e1.w};
      const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {sn.x, sn.y, sn.z, sn.w};
      // k leaves scaled by log2(e) / sqrt(128): the attention kernel's
      // scores are then directly the exponents of exp2.
      const float outscale = which ? K_SCORE_SCALE : 1.0f;
      float lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y0 = a[e] * rstd * ga[e] + ea[e];
        const float y1 = b[e] * rstd * gb[e] + eb[e];
        lo[e] = (y0 * cc[e] - y1 * ss[e]) * outscale;
        hi[e] = (y1 * cc[e] + y0 * ss[e]) * outscale;
      }
      *reinterpret_cast<uint2*>(base + d0) =
          make_uint2(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]));
      *reinterpret_cast<uint2*>(base + 64 + d0) =
          make_uint2(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
    }
  }

  // v: each thread transposes one 8 x 8 block (8 positions x 8 dims) in
  // registers -- output word k of column c takes half c%2 of word c/2 from
  // rows 2k and 2k+1 (one byte permute each) -- and stores 8 keys of each of
  // its 8 dims as 16-byte vectors.  Positions past the clip are zeros.
  // Key order inside each group of 16 columns: positions 0-3, 8-11, 4-7,
  // 12-15 of the group, so that 8 consecutive columns are the 8 keys one
  // lane supplies to a 32x32x16 MFMA whose other operand comes from the
  // accumulator layout of K Q^T (rows 4*(lane/32) + 8g + r).
  {
    const int rb = threadIdx.x >> 4;           // 16 blocks of 8 columns
    const int db = threadIdx.x & 15;           // 16 blocks of 8 dims
    if (rb * 8 < span) {
      uint4 rows[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int p = p0 + 16 * (rb >> 1) + 4 * (rb & 1) + (i & 3) + 8 * (i >> 2);
        rows[i] = (p < len) ? *reinterpret_cast<const uint4*>(qkv + (s0 + p) * (3 * D) + 2 * D +
                                                               h * DH + db * 8)
                            : make_uint4(0, 0, 0, 0);
      }
      bf16_t* dst = vt + ((int64_t)h * DH + db * 8) * ld_vt + vt_base[seq] + p0 + rb * 8;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t* ra = reinterpret_cast<const uint32_t*>(&rows[2 * k]);
          const uint32_t* rb2 = reinterpret_cast<const uint32_t*>(&rows[2 * k + 1]);
          w[k] = __builtin_amdgcn_perm(rb2[c >> 1], ra[c >> 1], sel);
        }
        *reinterpret_cast<uint4*>(dst + (int64_t)c * ld_vt) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
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
