// Variable-length bidirectional softmax attention for gfx950 (flash style:
// the score matrix never leaves registers).
//
// Method: ten heads of width 128 with full self-attention over each clip
// ("Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
// "How audio and speakers reach the language model"; the same page's section
// "Local encoder windows, recording-wide language context" notes that
// FlashAttention-style kernels avoid materialising the quadratic score matrix).
//
// Work split: a workgroup takes 128 queries of one clip and one head; each of
// its four wavefronts owns 32 queries and walks the clip's keys 64 at a time.
// Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16,
// so every lane holds 16 keys of one query: the running max and sum of the
// online softmax need one cross-lane exchange (lanes l and l ^ 32) per tile.
// The probabilities feed O^T += V^T P^T straight from registers; V arrives
// already transposed (per head [dim][key]) and is staged in LDS with its keys
// permuted inside each group of 16 so that a lane's eight operand keys are
// contiguous.  Keys past the clip end are masked to -inf in S; their V^T
// columns (up to the next multiple of 64) are zero.

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr int QB = 128;     // queries per workgroup (4 wavefronts x 32)
constexpr int KB = 64;      // keys per tile

// Position of key kappa (0..63) inside an LDS row of the V^T tile: within each
// group of 16 keys, blocks of 4 are stored in the order 0, 2, 1, 3.
__device__ __forceinline__ int vperm(int kappa) {
  const int blk = (kappa >> 2) & 3;
  const int nb = (blk == 1) ? 2 : (blk == 2 ? 1 : blk);
  return (kappa & ~15) | (nb << 2) | (kappa & 3);
}

__global__ __launch_bounds__(256) void attention_kernel(
    const bf16_t* __restrict__ qkv, const bf16_t* __restrict__ vt, int64_t ld_vt,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ vt_base,
    const int32_t* __restrict__ tile_seq,
    const int32_t* __restrict__ tile_q0, bf16_t* __restrict__ out) {
  __shared__ uint4 sK[KB * DH / 8];          // [key][16 chunks], swizzled
  __shared__ uint2 sV[DH * KB / 4];          // [dim][16 half-chunks], permuted+swizzled

  const int tile = blockIdx.x;
  const int h = blockIdx.y;
  const int seq = tile_seq[tile];
  const int64_t s0 = cu[seq];
  const int len = cu[seq + 1] - cu[seq];
  const int q0 = tile_q0[tile];
  const bf16_t* vbase = vt + (int64_t)h * DH * ld_vt + vt_base[seq];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // Q^T fragments for this lane's query, 8 k-steps of 16 dims.
  static_assert(QB == 4 * 32, "one 32-query block per wavefront");
  const int qi = q0 + wave * 32 + l32;
  bf16x8 qf[DH / 16];
  {
    const bool ok = qi < len;
    const bf16_t* qrow = qkv + (s0 + (ok ? qi : 0)) * (3 * D) + h * DH;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) {
      uint4 u = ok ? *reinterpret_cast<const uint4*>(qrow + s * 16 + lhi * 8) : make_uint4(0, 0, 0, 0);
      qf[s] = *reinterpret_cast<const bf16x8*>(&u);
    }
  }

  f32x16 acc_o[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc_o[i][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float scale = 0.08838834764831845f * 1.4426950408889634f;   // 1/sqrt(128) * log2(e)

  // Staging: 4 K chunks and 4 V^T chunks (16 B each) per thread per tile.
  uint4 rk[4], rv[4];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int key = c >> 4, kc = c & 15;
      const int kk = kv0 + key;
      rk[i] = (kk < len) ? *reinterpret_cast<const uint4*>(qkv + (s0 + kk) * (3 * D) + D + h * DH + kc * 8)
                         : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int d = c >> 3, kc = c & 7;
      // columns up to roundup(len, 64) exist and are zero past len
      rv[i] = *reinterpret_cast<const uint4*>(vbase + (int64_t)d * ld_vt + kv0 + kc * 8);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int key = c >> 4, kc = c & 15;
      sK[key * 16 + (kc ^ (key & 15))] = rk[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int d = c >> 3, kc = c & 7;
      // keys kc*8 .. kc*8+7 = two blocks of 4, each to its permuted slot
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int pos = vperm(kc * 8 + half * 4);          // multiple of 4
        const int chunk = pos >> 3, sub = (pos >> 2) & 1;  // 16-byte chunk, 8-byte half
        const int slot = ((chunk ^ (d & 7)) << 1) | sub;
        sV[d * 16 + slot] = half ? make_uint2(rv[i].z, rv[i].w) : make_uint2(rv[i].x, rv[i].y);
      }
    }
  };

  load_tile(0);
  for (int kv0 = 0; kv0 < len; kv0 += KB) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kv0 + KB < len) load_tile(kv0 + KB);

    // S^T for two blocks of 32 keys.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[kb][v] = 0.f;
#pragma unroll
      for (int s = 0; s < DH / 16; ++s) {
        const int key = kb * 32 + l32;
        const int chunk = 2 * s + lhi;
        const uint4 u = sK[key * 16 + (chunk ^ (key & 15))];
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(&u),
                                                           qf[s], sacc[kb], 0, 0, 0);
      }
    }

    // Online softmax over this tile (lane: one query, 32 of the 64 keys).
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kv0 + kb * 32 + 8 * (v >> 2) + 4 * lhi + (v & 3);
        const float sv = (key < len) ? sacc[kb][v] * scale : -INFINITY;
        sacc[kb][v] = sv;
        tmax = fmaxf(tmax, sv);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - m_new);
    float tsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = exp2f(sacc[kb][v] - m_new);
        sacc[kb][v] = p;
        tsum += p;
      }
    tsum += __shfl_xor(tsum, 32, 64);
    l_run = l_run * alpha + tsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc_o[i][v] *= alpha;

    // O^T += V^T P^T over four k-steps of 16 keys.
#pragma unroll
    for (int kk = 0; kk < KB / 16; ++kk) {
      const int kb = kk >> 1, v0 = (kk & 1) * 8;
      uint32_t pk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) pk[j] = pack_bf16x2(sacc[kb][v0 + 2 * j], sacc[kb][v0 + 2 * j + 1]);
      const bf16x8 pf = *reinterpret_cast<const bf16x8*>(pk);
#pragma unroll
      for (int db = 0; db < DH / 32; ++db) {
        const int d = db * 32 + l32;
        const int chunk = 2 * kk + lhi;
        const int slot = (chunk ^ (d & 7)) << 1;
        const uint2 a = sV[d * 16 + slot];
        const uint2 b = sV[d * 16 + slot + 1];
        const uint4 u = make_uint4(a.x, a.y, b.x, b.y);
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(&u),
                                                            pf, acc_o[db], 0, 0, 0);
      }
    }
  }

  if (qi >= len) return;
  const float inv = 1.0f / l_run;
  bf16_t* orow = out + (s0 + qi) * D + h * DH;
#pragma unroll
  for (int db = 0; db < DH / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * lhi;
      *reinterpret_cast<uint2*>(orow + d) =
          make_uint2(pack_bf16x2(acc_o[db][4 * g] * inv, acc_o[db][4 * g + 1] * inv),
                     pack_bf16x2(acc_o[db][4 * g + 2] * inv, acc_o[db][4 * g + 3] * inv));
    }
}

}  // namespace

hipError_t launch_attention(const bf16_t* qkv, const bf16_t* vt, int64_t ld_vt,
                            const int32_t* cu_seq, const int32_t* vt_base, const int32_t* tile_seq,
                            const int32_t* tile_q0, int n_tiles, bf16_t* out,
                            hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  attention_kernel<<<dim3(n_tiles, H), dim3(256), 0, stream>>>(qkv, vt, ld_vt, cu_seq, vt_base,
                                                               tile_seq, tile_q0, out);
  return hipGetLastError();
}

}  // namespace enc
