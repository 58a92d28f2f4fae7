// Row-wise kernels for gfx950: LayerNorm (pre-norm and final), fused QK
// normalisation + rotary embedding, and the element conversions used when
// weights are copied in.
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

#include <algorithm>
#include <cmath>

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

// LayerNorm with E4M3 output (the FP8 linear maps' input): codes of
// LN(x) * g + b times out_scale, saturated at +-448.
__global__ __launch_bounds__(256) void layernorm_fp8_kernel(const float* __restrict__ x,
                                                            const float* __restrict__ g,
                                                            const float* __restrict__ b,
                                                            float out_scale,
                                                            uint8_t* __restrict__ y8,
                                                            int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  float4 o[5];
  ln_row_1280(x + r * D, g, b, lane, o);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int c = (i * 64 + lane) * 4;
    *reinterpret_cast<uint32_t*>(y8 + r * D + c) =
        pack_fp8x4(o[i].x * out_scale, o[i].y * out_scale, o[i].z * out_scale,
                   o[i].w * out_scale);
  }
}

// Largest magnitude of a bf16 tensor, merged into *amax (calibration).
__global__ __launch_bounds__(256) void amax_bf16_kernel(const bf16_t* __restrict__ x, int64_t n8,
                                                        float* __restrict__ amax) {
  __shared__ float part[4];
  float m = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m = fmaxf(m, fabsf(__uint_as_float(w[k] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(w[k] & 0xffff0000u)));
    }
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
  }
}

// Per-tensor E4M3 codes of a bf16 matrix under s = amax / 448.
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const bf16_t* __restrict__ w,
                                                           int64_t n8,
                                                           const float* __restrict__ amax,
                                                           float* __restrict__ scale,
                                                           uint8_t* __restrict__ q) {
  const float a = *amax;
  const float s = a > 0.0f ? a / E4M3_MAX : 1.0f;
  const float r = 1.0f / s;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i == 0) *scale = s;
  if (i >= n8) return;
  const uint4 v = reinterpret_cast<const uint4*>(w)[i];
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    out[k] = pack_fp8x4(__uint_as_float(u[2 * k] << 16) * r,
                        __uint_as_float(u[2 * k] & 0xffff0000u) * r,
                        __uint_as_float(u[2 * k + 1] << 16) * r,
                        __uint_as_float(u[2 * k + 1] & 0xffff0000u) * r);
  reinterpret_cast<uint2*>(q)[i] = make_uint2(out[0], out[1]);
}

__global__ void fill_f32_kernel(float* __restrict__ p, float v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void final_norm_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ b,
                                                         const int32_t* __restrict__ cu,
                                                         const int32_t* __restrict__ src_rows,
                                                         int batch, int64_t p_max,
                                                         bf16_t* __restrict__ out) {
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
  const int64_t row = (int64_t)cu[bi] + p;
  float4 o[5];
  ln_row_1280(x + (src_rows ? (int64_t)src_rows[row] : row) * D, g, b, lane, o);
#pragma unroll
  for (int i = 0; i < 5; ++i)
    *reinterpret_cast<uint2*>(dst + (i * 64 + lane) * 4) =
        make_uint2(pack_bf16x2(o[i].x, o[i].y), pack_bf16x2(o[i].z, o[i].w));
}

// QK-norm layout: 8 lanes per (row, head); lane j holds dims 8j..8j+7 and
// 64+8j..64+8j+7, i.e. eight whole rotation pairs, so the rotation is local,
// every access is a 16-byte vector and a wavefront's access covers whole
// 128-byte lines; the statistics reduce over the 8 lanes.  The plan's tiles
// are QK_ROWS positions; a workgroup takes a quarter of one.
constexpr int QK_ROWS = 128;
constexpr int QK_HEAD_GROUPS = 5;   // measured: 2 heads per group for 10 heads

__device__ __forceinline__ void unpack8(const uint4 u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// q and k of 32 positions (8 per wavefront, 8 lanes per position) over all
// heads: normalise, rotate, scale k (in place).  The QK-norm gains and biases
// (shared by the heads) and the position's rotation table row are loaded once
// and serve every head; the next head's q and k are loaded while the current
// one is computed.
// HALF = half the head width (rotation pairs (i, i + HALF)): 64 for the
// encoder's heads, 40 for the timestamp adapter's; heads are packed at their
// width.  ldq: row stride of qkv, hd: offset of the k block within a row
// (heads x 2 HALF), kscale: factor on k.
template <int HALF>
__device__ __forceinline__ void qk_rows(bf16_t* __restrict__ qkv, int64_t ldq, int hd, int h0,
                                        int h1, int64_t s0, int len, int p, int lane,
                                        const float* __restrict__ qg,
                                        const float* __restrict__ qb, const float* __restrict__ kg,
                                        const float* __restrict__ kb,
                                        const float* __restrict__ rope_cos,
                                        const float* __restrict__ rope_sin, float kscale) {
  if (h0 >= h1) return;          // an empty group (heads not divisible)
  constexpr float INV_DH = 1.0f / (2 * HALF);
  const int sub = lane & 7;     // dims 8 sub .. + 7 and HALF + 8 sub .. + 7
  const bool act = sub < HALF / 8;   // lanes past the head width idle
  const int d0 = (act ? sub : 0) * 8;
  const bool live = p < len;    // uniform over the 8 lanes of the row
  const int pl = live ? p : 0;  // rows past the clip read row 0 and store nothing
  float gq[2][8], bq[2][8], gk[2][8], bk[2][8];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gq[hh][e] = qg[hh * HALF + d0 + e];
      bq[hh][e] = qb[hh * HALF + d0 + e];
      gk[hh][e] = kg[hh * HALF + d0 + e];
      bk[hh][e] = kb[hh * HALF + d0 + e];
    }
  float cs[8], sn[8];
  {
    const float4 c0 = *reinterpret_cast<const float4*>(rope_cos + (int64_t)pl * HALF + d0);
    const float4 c1 = *reinterpret_cast<const float4*>(rope_cos + (int64_t)pl * HALF + d0 + 4);
    const float4 s0v = *reinterpret_cast<const float4*>(rope_sin + (int64_t)pl * HALF + d0);
    const float4 s1v = *reinterpret_cast<const float4*>(rope_sin + (int64_t)pl * HALF + d0 + 4);
    cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w;
    cs[4] = c1.x; cs[5] = c1.y; cs[6] = c1.z; cs[7] = c1.w;
    sn[0] = s0v.x; sn[1] = s0v.y; sn[2] = s0v.z; sn[3] = s0v.w;
    sn[4] = s1v.x; sn[5] = s1v.y; sn[6] = s1v.z; sn[7] = s1v.w;
  }
  bf16_t* row = qkv + (s0 + pl) * ldq + d0;
  // u[0..1]: q dims d0.. and HALF + d0..; u[2..3]: the same of k
  auto load = [&](int h, uint4 (&u)[4]) __attribute__((always_inline)) {
    const bf16_t* base = row + h * (2 * HALF);
    u[0] = *reinterpret_cast<const uint4*>(base);
    u[1] = *reinterpret_cast<const uint4*>(base + HALF);
    u[2] = *reinterpret_cast<const uint4*>(base + hd);
    u[3] = *reinterpret_cast<const uint4*>(base + hd + HALF);
  };
  uint4 cur[4], nxt[4];
  load(h0, cur);
#pragma unroll 1
  for (int h = h0; h < h1; ++h) {
    if (h + 1 < h1) load(h + 1, nxt);
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      float a[8], b[8];
      unpack8(cur[2 * which], a);
      unpack8(cur[2 * which + 1], b);
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += a[e] + b[e];
      if (!act) sum = 0.f;
      sum = group8_sum(sum);
      const float mean = sum * INV_DH;
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] -= mean;
        b[e] -= mean;
        sq += a[e] * a[e] + b[e] * b[e];
      }
      if (!act) sq = 0.f;
      sq = group8_sum(sq);
      const float rstd = rsqrtf(sq * INV_DH + LN_EPS);
      // k leaves scaled by log2(e) / sqrt(head width): the attention
      // kernel's scores are then directly the exponents of exp2.
      const float outscale = which ? kscale : 1.0f;
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float y0[2], y1[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float ga = which ? gk[0][e + t] : gq[0][e + t];
          const float gb = which ? gk[1][e + t] : gq[1][e + t];
          const float ea = which ? bk[0][e + t] : bq[0][e + t];
          const float eb = which ? bk[1][e + t] : bq[1][e + t];
          const float x0 = a[e + t] * rstd * ga + ea;
          const float x1 = b[e + t] * rstd * gb + eb;
          y0[t] = (x0 * cs[e + t] - x1 * sn[e + t]) * outscale;
          y1[t] = (x1 * cs[e + t] + x0 * sn[e + t]) * outscale;
        }
        lo[e / 2] = pack_bf16x2(y0[0], y0[1]);
        hi[e / 2] = pack_bf16x2(y1[0], y1[1]);
      }
      if (live && act) {
        bf16_t* base = row + which * hd + h * (2 * HALF);
        *reinterpret_cast<uint4*>(base) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        *reinterpret_cast<uint4*>(base + HALF) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) cur[t] = nxt[t];
  }
}

template <int HALF>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    bf16_t* __restrict__ qkv, const int4* __restrict__ tile_info,
    const float* __restrict__ qg, const float* __restrict__ qb, const float* __restrict__ kg,
    const float* __restrict__ kb, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, int hd, int n_heads, int hgroups, float kscale) {
  const int64_t ldq = 3 * (int64_t)hd;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // Block b: q and k of a quarter tile (32 positions) for one of `hgroups`
  // groups of heads.
  constexpr int QUARTERS = QK_ROWS / 32;
  const int hg = blockIdx.x % hgroups;
  const int tq = blockIdx.x / hgroups;
  const int t = tq / QUARTERS;
  const int4 ti = tile_info[t];   // first row, length, first position
  const int len = ti.y;
  const int p = ti.z + (tq % QUARTERS) * 32 + wave * 8 + (lane >> 3);
  if (__builtin_amdgcn_readfirstlane(p - (lane >> 3)) >= len) return;   // no live row
  const int per = (n_heads + hgroups - 1) / hgroups;
  qk_rows<HALF>(qkv, ldq, hd, hg * per, min(n_heads, (hg + 1) * per), ti.x, len, p, lane, qg,
                qb, kg, kb, rope_cos, rope_sin, kscale);
}

// dst[r, :] = src[rows[r], :] for rows of 1024 bf16 (one wavefront per row,
// 32 bytes per lane).
__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16_t* __restrict__ src,
                                                          const int32_t* __restrict__ rows,
                                                          int64_t n, bf16_t* __restrict__ dst) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const uint4* s = reinterpret_cast<const uint4*>(src + (int64_t)rows[r] * DIN) + lane * 2;
  uint4* d = reinterpret_cast<uint4*>(dst + r * DIN) + lane * 2;
  const uint4 a = s[0], b2 = s[1];
  d[0] = a;
  d[1] = b2;
}

// Speaker-activity fusion, section "How audio and speakers reach the language
// model": the activity of the 8 speaker slots is thresholded at 0.5 (1 where
// > 0.5), normalised by a LayerNorm over the slots, mapped to width 1280 by a
// fixed sinusoidal table and added to the encoder states.  Row r of the
// clip-packed output: y = LN_f(x[s]) + sum_j n_j tab[j], n = LN_spk(act[r] > 0.5),
// s = src_rows ? src_rows[r] : r; bf16 output (the connector GEMM's operand).
// The 8 x 1280 table is staged in LDS once per workgroup of FUSE_ROWS rows;
// each lane then reads its own 20 columns of the 8 rows as 16-byte vectors.
constexpr int FUSE_ROWS = 32;

__global__ __launch_bounds__(256) void speaker_fuse_kernel(
    const float* __restrict__ x, const float* __restrict__ g, const float* __restrict__ b,
    const int32_t* __restrict__ src_rows, int64_t rows, const float* __restrict__ act,
    const float* __restrict__ sg, const float* __restrict__ sb, const float* __restrict__ tab,
    bf16_t* __restrict__ out) {
  __shared__ float4 stab[NSPK * D / 4];
  for (int i = threadIdx.x; i < NSPK * D / 4; i += 256)
    stab[i] = reinterpret_cast<const float4*>(tab)[i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int k = 0; k < FUSE_ROWS / 4; ++k) {
    const int64_t r = (int64_t)blockIdx.x * FUSE_ROWS + k * 4 + wave;
    if (r >= rows) break;
    float4 o[5];
    ln_row_1280(x + (src_rows ? (int64_t)src_rows[r] : r) * D, g, b, lane, o);
    const float4 a0 = *reinterpret_cast<const float4*>(act + r * NSPK);
    const float4 a1 = *reinterpret_cast<const float4*>(act + r * NSPK + 4);
    float n[NSPK] = {a0.x > 0.5f ? 1.f : 0.f, a0.y > 0.5f ? 1.f : 0.f, a0.z > 0.5f ? 1.f : 0.f,
                     a0.w > 0.5f ? 1.f : 0.f, a1.x > 0.5f ? 1.f : 0.f, a1.y > 0.5f ? 1.f : 0.f,
                     a1.z > 0.5f ? 1.f : 0.f, a1.w > 0.5f ? 1.f : 0.f};
    float mean = 0.f;
#pragma unroll
    for (int j = 0; j < NSPK; ++j) mean += n[j];
    mean *= 1.0f / NSPK;
    float var = 0.f;
#pragma unroll
    for (int j = 0; j < NSPK; ++j) {
      n[j] -= mean;
      var += n[j] * n[j];
    }
    const float rstd = rsqrtf(var * (1.0f / NSPK) + LN_EPS);
#pragma unroll
    for (int j = 0; j < NSPK; ++j) n[j] = n[j] * rstd * sg[j] + sb[j];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
#pragma unroll
      for (int j = 0; j < NSPK; ++j) {
        const float4 t = stab[j * (D / 4) + i * 64 + lane];
        o[i].x = fmaf(n[j], t.x, o[i].x);
        o[i].y = fmaf(n[j], t.y, o[i].y);
        o[i].z = fmaf(n[j], t.z, o[i].z);
        o[i].w = fmaf(n[j], t.w, o[i].w);
      }
      *reinterpret_cast<uint2*>(out + r * D + (i * 64 + lane) * 4) =
          make_uint2(pack_bf16x2(o[i].x, o[i].y), pack_bf16x2(o[i].z, o[i].w));
    }
  }
}

// Log-softmax of one row per workgroup: the row (up to LSM_MAX values) is
// read once into registers (24 float4 per thread), then its maximum, the sum
// of exp(z - max) and the output z - max - log(sum) come from the registers.
constexpr int LSM_CHUNKS = 24;
constexpr int LSM_MAX = LSM_CHUNKS * 4 * 256;

__device__ __forceinline__ float block_reduce4(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  __syncthreads();   // red is reused
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]))
                : (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void log_softmax_kernel(const float* __restrict__ z,
                                                          int64_t ldz, int n,
                                                          float* __restrict__ out) {
  __shared__ float red[4];
  const float* zr = z + (int64_t)blockIdx.x * ldz;
  float4 v[LSM_CHUNKS];
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < LSM_CHUNKS; ++c) {
    const int e = (threadIdx.x + 256 * c) * 4;
    // ldz is a multiple of 4, so a chunk that starts before n lies in the row
    v[c] = e < n ? *reinterpret_cast<const float4*>(zr + e)
                 : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    if (e + 1 >= n) v[c].y = -INFINITY;
    if (e + 2 >= n) v[c].z = -INFINITY;
    if (e + 3 >= n) v[c].w = -INFINITY;
    m = fmaxf(m, fmaxf(fmaxf(v[c].x, v[c].y), fmaxf(v[c].z, v[c].w)));
  }
  m = block_reduce4(m, red, true);
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < LSM_CHUNKS; ++c)
    sum += (__expf(v[c].x - m) + __expf(v[c].y - m)) + (__expf(v[c].z - m) + __expf(v[c].w - m));
  const float lse = m + __logf(block_reduce4(sum, red, false));
  float* orow = out + (int64_t)blockIdx.x * n;
#pragma unroll
  for (int c = 0; c < LSM_CHUNKS; ++c) {
    const int e = (threadIdx.x + 256 * c) * 4;
    if (e < n) orow[e] = v[c].x - lse;
    if (e + 1 < n) orow[e + 1] = v[c].y - lse;
    if (e + 2 < n) orow[e + 2] = v[c].z - lse;
    if (e + 3 < n) orow[e + 3] = v[c].w - lse;
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

hipError_t launch_layernorm_fp8(const float* x, const float* g, const float* b, float out_scale,
                                uint8_t* y8, int64_t rows, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  layernorm_fp8_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(
      x, g, b, out_scale, y8, rows);
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const bf16_t* x, int64_t n, float* amax, hipStream_t stream) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const int64_t n8 = n / 8;
  const unsigned grid = (unsigned)std::min<int64_t>((n8 + 255) / 256, 2048);
  amax_bf16_kernel<<<dim3(grid), dim3(256), 0, stream>>>(x, n8, amax);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const bf16_t* w, int64_t n, const float* amax, float* scale,
                               uint8_t* q, hipStream_t stream) {
  if (n % 8 != 0 || n == 0) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  quantize_fp8_kernel<<<dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream>>>(w, n8, amax,
                                                                                   scale, q);
  return hipGetLastError();
}

hipError_t launch_log_softmax(const float* z, int64_t ldz, int64_t rows, int n, float* out,
                              hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (n < 1 || n > LSM_MAX || ldz < n || ldz % 4 != 0 || rows > 0x7fffffff)
    return hipErrorInvalidValue;
  log_softmax_kernel<<<dim3((unsigned)rows), dim3(256), 0, stream>>>(z, ldz, n, out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  fill_f32_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(p, v, n);
  return hipGetLastError();
}

hipError_t launch_final_norm(const float* x, const float* g, const float* b, const int32_t* cu_seq,
                             const int32_t* src_rows,
                             int batch, int64_t p_max, bf16_t* out, hipStream_t stream) {
  const int64_t rows = (int64_t)batch * p_max;
  if (rows == 0) return hipSuccess;
  final_norm_kernel<<<dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream>>>(
      x, g, b, cu_seq, src_rows, batch, p_max, out);
  return hipGetLastError();
}

hipError_t launch_speaker_fuse(const float* x, const float* g, const float* b,
                               const int32_t* src_rows, int64_t rows, const float* act,
                               const float* spk_g, const float* spk_b, const float* spk_tab,
                               bf16_t* out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  speaker_fuse_kernel<<<dim3((unsigned)((rows + FUSE_ROWS - 1) / FUSE_ROWS)), dim3(256), 0,
                        stream>>>(x, g, b, src_rows, rows, act, spk_g, spk_b, spk_tab, out);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const bf16_t* src, const int32_t* rows, int64_t n, bf16_t* dst,
                              hipStream_t stream) {
  if (n == 0) return hipSuccess;
  gather_rows_kernel<<<dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream>>>(src, rows, n, dst);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(bf16_t* qkv, const int32_t* tile_info, int n_tiles, int n_heads,
                              int head_dim, const float* qg, const float* qb, const float* kg,
                              const float* kb, const float* rope_cos, const float* rope_sin,
                              hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  if (n_heads < 1) return hipErrorInvalidValue;
  const int hd = n_heads * head_dim;
  // log2(e) / sqrt(head width)
  const float kscale = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  // the heads are split into QK_HEAD_GROUPS groups, one block per group and
  // quarter tile (the gains and the rotation table row are loaded once per
  // group)
  const int hgroups = std::min(n_heads, QK_HEAD_GROUPS);
  const int64_t blocks = (int64_t)n_tiles * (QK_ROWS / 32) * hgroups;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  if (head_dim == DH)
    qknorm_rope_kernel<DH / 2><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        qkv, reinterpret_cast<const int4*>(tile_info), qg, qb, kg, kb, rope_cos, rope_sin, hd,
        n_heads, hgroups, kscale);
  else if (head_dim == 80)
    qknorm_rope_kernel<40><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        qkv, reinterpret_cast<const int4*>(tile_info), qg, qb, kg, kb, rope_cos, rope_sin, hd,
        n_heads, hgroups, kscale);
  else
    return hipErrorInvalidValue;
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
