// Variable-length bidirectional softmax attention for gfx950 (flash style:
// the score matrix never leaves registers).
//
// Method: ten heads of width 128 with full self-attention over each clip
// ("Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
// "How audio and speakers reach the language model"; the same page's section
// "Local encoder windows, recording-wide language context" notes that
// FlashAttention-style kernels avoid materialising the quadratic score matrix).
// The timestamp adapter's sixteen heads of width 80 run in the same kernel.
//
// Work split: a workgroup of four wavefronts takes 128 queries of one clip
// and one head, 32 queries per wavefront.  (Two wavefronts of 64 queries, in
// which every K or V^T fragment read from LDS feeds two MFMAs, need twice the
// accumulator registers and leave one wavefront per SIMD; with 32 queries two
// wavefronts share each SIMD and cover each other's load waits, which
// measured faster from 5 s clips to one hour.)  Scores are
// computed transposed, S^T = K Q^T, so a lane holds 16 keys of one query per
// 32-key block: the softmax needs one cross-lane exchange (lanes l, l ^ 32)
// per tile for the maximum and none for the sum.  Probabilities feed
// O^T += V^T P^T straight from registers.  V stays in the qkv rows as the QKV
// product wrote it ([key][dim]); its V^T operands come from the row-major LDS
// tile through the transposing LDS read (ds_read_b64_tr_b16), whose addresses
// also pick the keys in the order of the probabilities' accumulator layout.
//
// Long sequences whose work items would leave most of a last wave of
// workgroups idle cut each item's keys into runs and add the runs' partial
// sums in attention_combine_kernel (see launch_attention).
//
// Pipeline: K goes global -> LDS in 32-key units (a ring of four) and V in
// 64-key tiles (two buffers) by direct loads (global_load_lds, 16 bytes per
// lane, swizzle applied on the global side), one barrier per 64 keys.  The
// scores of unit u + 1 are issued to the matrix cores in the same basic block
// as unit u's exponentials and products with V, so the VALU work of the
// softmax overlaps the MFMAs.
//
// Softmax reference.  QK-norm bounds every score: after LayerNorm a head
// vector of width w has norm at most max|gain| * sqrt(w) + |bias|, so |q.k| is bounded
// by the product of the two norms.  When the launcher is told that this bound
// keeps scores * log2(e) / sqrt(w) within +-64 (kFixedRef), probabilities
// are exp2 of the scaled scores against a fixed reference of 0: no running
// maximum, no rescaling.  Each probability lies in [2^-64, 2^64], so a row
// sum over at most 90,000 keys stays below 2^81, and an output accumulator
// below 2^81 * max|v|: fp32 (to 2^128) holds both unless |v| exceeds 2^47,
// which a bf16 product of LayerNorm outputs and 0.02-scale weights cannot
// approach.  Otherwise the
// running maximum is kept lazily: the accumulators are rescaled only when a
// query's unit maximum exceeds it by more than 8 (log2 units); in between,
// probabilities are taken against the stale maximum (they stay below 2^8),
// which leaves the normalised result unchanged.
//
// Keys past the clip end: their K rows (read from whatever follows in the qkv
// buffer, which has 64 rows of slack) are masked to -inf by a select in the
// clip's last tile; their V rows repeat the clip's last row (probability 0).

#include <algorithm>
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr int QTILE = 128;             // queries per workgroup (the plan's tiles)
constexpr int KT = 64;                 // keys per V tile
constexpr int KU = 32;                 // keys per K unit (one score block)
constexpr int KU_BYTES = KU * DH * 2;  // 8 KB
constexpr int VT_BYTES = KT * DH * 2;  // 16 KB
constexpr int QB = 1;                  // 32-query blocks per wavefront
constexpr int QPW = 32 * QB;           // queries per wavefront
constexpr int NW = QTILE / QPW;        // wavefronts per workgroup
constexpr int KP = 8 / NW;             // 1-KB pieces of a K unit per wavefront
constexpr int VP = 16 / NW;            // 1-KB pieces of a V tile per wavefront

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 16 bytes per lane from g to LDS byte address lds + 16 * lane (lds is
// wave-uniform).  Written in asm so that the compiler does not track it: it
// would otherwise wait for these loads before every LDS read it cannot prove
// disjoint.  Callers wait with lds_loads_wait() before the barrier that
// publishes the data.  M0 is not otherwise used by this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void lds_loads_wait() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// HW: head width, 128 (the encoder) or 80 (the timestamp adapter).  Heads
// are packed at their own width in the qkv rows; in LDS every key row keeps
// 16 chunks of 8 dims, of which a narrower head fills the first HW / 8.
// Key splits (fixed reference only): with splits > 1 the keys of a clip are
// cut into runs of t_split 64-key tiles, item i of the launch takes run
// i % splits of work item i / splits, and instead of the normalised output
// it writes its unnormalised sums O (fp32, [split][row][head][HW]) and row
// sums l ([split][row][head]) to opart / lpart; against a fixed reference
// the partial sums of the runs add up to those of the whole clip
// (attention_combine_kernel).
template <bool kFixedRef, int HW>
__global__ __launch_bounds__(64 * NW) void attention_kernel(
    const bf16_t* __restrict__ qkv, const int4* __restrict__ tile_info, int n_tiles,
    int n_items, void* __restrict__ out, float out_scale, int hd, int splits, int t_split,
    float* __restrict__ opart, float* __restrict__ lpart, int64_t part_rows) {
  static_assert(HW % 16 == 0 && HW <= DH, "head width");
  constexpr int KS = HW / 16;          // 16-dim steps of the scores
  constexpr int NDB = (HW + 31) / 32;  // 32-dim blocks of the output
  constexpr int NCH = HW / 8;          // 16-byte chunks of a head row
  // K in a ring of four 32-key units, V in two 64-key tiles.
  __shared__ uint4 sK[4][KU * DH / 8];   // [key][16 chunks of 8 dims], swizzled
  __shared__ uint4 sV[2][KT * DH / 8];   // [key][16 chunks of 8 dims], swizzled

  // Hardware block b runs on XCD b % 8; XCD x takes items [x * per, x * per +
  // per) so that the workgroups resident on one XCD walk the same head's keys.
  const int per = gridDim.x >> 3;
  const int item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (item >= n_items) return;
  const int split = item % splits;
  const int h = item / splits / n_tiles;
  const int tile = item / splits - h * n_tiles;
  const int4 ti = tile_info[tile];   // first row, length, first query
  const int64_t s0 = ti.x;
  const int len = ti.y;              // queries (and keys of the whole clip)
  const int q0 = ti.z;
  const int n_heads = hd / HW;
  // keys of this run: [kfirst, kfirst + klen) of the clip
  const int kfirst = split * t_split * KT;
  const int klen = splits > 1 ? min(len - kfirst, t_split * KT) : len;
  if (klen <= 0) {
    // an empty run (a clip shorter than the longest): zero partial sums
    for (int e = threadIdx.x; e < QTILE * (HW + 1); e += 64 * NW) {
      const int r = e / (HW + 1), d = e - r * (HW + 1);
      const int q = q0 + r;
      if (q >= len) continue;
      const int64_t pr = ((int64_t)split * part_rows + s0 + q) * n_heads + h;
      if (d < HW) opart[pr * HW + d] = 0.f;
      else lpart[pr] = 0.f;
    }
    return;
  }
  const int nkt = (klen + KT - 1) / KT;   // 64-key tiles
  const int nku = 2 * nkt;                // 32-key units

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // Q^T fragments: query block qb, 16-dim step s.
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = q0 + wave * QPW + qb * 32 + l32;
    const bool ok = q < len;
    const bf16_t* qrow = qkv + (s0 + (ok ? q : 0)) * (3 * hd) + h * HW + lhi * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 u = ok ? *reinterpret_cast<const uint4*>(qrow + s * 16) : make_uint4(0, 0, 0, 0);
      qf[qb][s] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // Direct loads, in 1-KB pieces of four key rows (lane -> key 4i + lane/16,
  // LDS chunk lane%16 of the row).  A K unit is eight pieces, LDS chunk c of
  // key k holding global chunk c ^ (k%16); this wave loads pieces
  // KP*wave..KP*wave+KP-1.  A V tile is sixteen pieces, LDS chunk c of key k
  // holding global chunk c ^ 4(k%4); this wave loads VP*wave..VP*wave+VP-1.
  // Offsets are bytes from the unit's / tile's first key row.  A narrower
  // head has fewer chunks than the LDS row: lanes whose global chunk lies
  // past it load chunk - 8 of the same row instead (finite data in LDS chunks
  // that the scores never read and that only reach output dims >= HW).
  auto in_head = [](int c) { return NCH == 16 || c < NCH ? c : c - 8; };
  uint32_t koff[KP], vchunk[VP];
#pragma unroll
  for (int t = 0; t < KP; ++t) {
    const int key = (wave * KP + t) * 4 + (lane >> 4);
    koff[t] = (uint32_t)(key * (3 * hd * 2) + in_head((lane & 15) ^ (key & 15)) * 16);
  }
#pragma unroll
  for (int t = 0; t < VP; ++t) {
    const int key = (wave * VP + t) * 4 + (lane >> 4);
    vchunk[t] = (uint32_t)(in_head((lane & 15) ^ (4 * (key & 3))) * 16);
  }
  const char* kbase =
      reinterpret_cast<const char*>(qkv + (s0 + kfirst) * (3 * hd) + hd + h * HW);
  const char* vbase =
      reinterpret_cast<const char*>(qkv + (s0 + kfirst) * (3 * hd) + 2 * hd + h * HW);
  const uint32_t k_lds = (uint32_t)(uintptr_t)(lds_void*)&sK[0][0] + wave * KP * 1024;
  const uint32_t v_lds = (uint32_t)(uintptr_t)(lds_void*)&sV[0][0] + wave * VP * 1024;
  // K unit u into ring slot u % 4.  Units past the clip's last one re-load
  // the last unit into a slot that is never read again (no branch).
  auto issue_k = [&](int u) __attribute__((always_inline)) {
    const char* g = kbase + (int64_t)min(u, nku - 1) * KU * (3 * hd * 2);
    const uint32_t l = k_lds + (u & 3) * KU_BYTES;
#pragma unroll
    for (int t = 0; t < KP; ++t) dma16(g + koff[t], l + t * 1024);
  };
  // V tile j (keys 64 j ..) into buffer j % 2.  Keys past the run take the
  // run's last row: their probability is exactly 0, and a row of the clip is
  // finite whatever lies beyond it.
  auto issue_v = [&](int j) __attribute__((always_inline)) {
    const uint32_t l = v_lds + (j & 1) * VT_BYTES;
#pragma unroll
    for (int t = 0; t < VP; ++t) {
      const int key = min(j * KT + (wave * VP + t) * 4 + (lane >> 4), klen - 1);
      dma16(vbase + (int64_t)key * (3 * hd * 2) + vchunk[t], l + t * 1024);
    }
  };

  // Scores arrive in log2 units (k was scaled by log2(e) / sqrt(HW)).
  float m_run[QB], l_run[QB];     // running maxima; this lane's partial row sums
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  f32x16 O[NDB][QB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[db][qb][v] = 0.f;

  f32x16 SA[QB], SB[QB];   // scores of one 32-key unit, per query block

  const int kx = lhi ^ (l32 & 15);          // K chunk swizzle of this lane
  // V^T operands come from the row-major V tile through ds_read_b64_tr_b16:
  // within each group of 16 lanes, lane 4a + e receives element e of the
  // 8-byte chunks addressed by lanes a, a + 4, a + 8, a + 12.  Lane 4j + a
  // of group g addresses key row 4 (g/2) + j (+ 8 for the second read) at
  // dims 16 (g%2) + 4a .. + 3 of the 32-dim block, so lane l receives dim
  // l%32 of keys 4 lhi + 0..3 and 8 + 4 lhi + 0..3 -- the keys whose
  // probabilities it holds in the accumulator layout of K Q^T (rows
  // 8 (v/4) + 4 lhi + v%4).
  const int tr_j = (lane & 15) >> 2;
  const uint32_t tr_off =
      (uint32_t)((4 * (lane >> 5) + tr_j) * (DH * 2) + ((((lane >> 4) & 1) * 2 + ((lane & 3) >> 1)) << 4) +
                 ((lane & 1) << 3));
  const uint32_t v_lds0 = (uint32_t)(uintptr_t)(lds_void*)&sV[0][0];

  // S^T of unit u: 8 k-steps x 2 query blocks.
  auto qk = [&](f32x16 (&S)[QB], int u) __attribute__((always_inline)) {
    const uint4* sk = sK[u & 3];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int v = 0; v < 16; ++v) S[qb][v] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, sk[l32 * 16 + ((2 * s) ^ kx)]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][s], S[qb], 0, 0, 0);
    }
  };

  // Mask keys past the clip (unit u).  With a running maximum: take the
  // unit's maximum and rescale the accumulators if some query's maximum grew
  // by more than 8.
  auto decide = [&](f32x16 (&S)[QB], int u) __attribute__((always_inline)) {
    const int kv0 = u * KU;
    if (kv0 + KU > klen) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = kv0 + 8 * (v >> 2) + 4 * lhi + (v & 3);
          S[qb][v] = key < klen ? S[qb][v] : -INFINITY;
        }
    }
    if constexpr (!kFixedRef) {
      float mx[QB];
      bool grew = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float m = S[qb][0];
#pragma unroll
        for (int v = 1; v < 16; ++v) m = fmaxf(m, S[qb][v]);
        mx[qb] = fmaxf(m, __shfl_xor(m, 32, 64));
        grew = grew || mx[qb] > m_run[qb] + 8.0f;
      }
      if (__any(grew)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float mn = fmaxf(m_run[qb], mx[qb]);
          const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mn);
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) O[db][qb][v] *= alpha;
          m_run[qb] = mn;
        }
      }
    }
  };

  // Probabilities of one unit and O^T += V^T P^T over its two 16-key steps
  // (kk0, kk0 + 1 of V tile j).  Row sums take the bf16 probabilities the
  // products use (one dot2 per pair).
  auto expv = [&](f32x16 (&S)[QB], int j, int kk0) __attribute__((always_inline)) {
    const uint32_t sv = v_lds0 + (j & 1) * VT_BYTES;
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float nm = kFixedRef ? 0.f : -m_run[qb];
        uint32_t pk[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float p0 = S[qb][half * 8 + 2 * jj], p1 = S[qb][half * 8 + 2 * jj + 1];
          if constexpr (!kFixedRef) {
            p0 += nm;
            p1 += nm;
          }
          pk[jj] = pack_bf16x2(__builtin_amdgcn_exp2f(p0), __builtin_amdgcn_exp2f(p1));
          l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[jj]), ones,
                                                      l_run[qb], false);
        }
        pf[qb] = __builtin_bit_cast(bf16x8, pk);
      }
      const int kk = kk0 + half;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // chunk 4 db + q of key row k sits at 4 (db ^ (k%4)) + q, and k%4 = tr_j
        const uint32_t at = sv + kk * 16 * (DH * 2) + tr_off + ((db ^ tr_j) << 6);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)at);
        const v4i16 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(at + 8 * DH * 2));
        const bf16x8 vf =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          O[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb], O[db][qb], 0, 0, 0);
      }
    }
  };

  // Prologue: K units 0..2 and V tile 0; scores of unit 0.
  issue_k(0);
  issue_k(1);
  issue_k(2);
  issue_v(0);
  lds_loads_wait();
  __syncthreads();
  qk(SA, 0);
  decide(SA, 0);

  // Tile j (not the last one): units 2j, 2j+1 go through softmax and V while
  // the scores of units 2j+1 and 2j+2 are computed.  K units 2j+1, 2j+2 and
  // V tile j were loaded during the previous step; this step loads K units
  // 2j+3, 2j+4 into the slots of 2j-1, 2j and V tile j+1 into the buffer
  // of tile j-1, all read before the barrier.
#pragma unroll 1
  for (int j = 0; j + 1 < nkt; ++j) {
    lds_loads_wait();
    __syncthreads();
    issue_k(2 * j + 3);
    issue_k(2 * j + 4);
    issue_v(j + 1);
    qk(SB, 2 * j + 1);
    expv(SA, j, 0);
    if constexpr (!kFixedRef) decide(SB, 2 * j + 1);
    qk(SA, 2 * j + 2);
    expv(SB, j, 2);
    // Unit 2j+2 may lie in the last tile: with a fixed reference its mask is
    // applied below; a running maximum needs it now.
    if constexpr (!kFixedRef) decide(SA, 2 * j + 2);
  }

  // Last tile.
  {
    const int j = nkt - 1;
    lds_loads_wait();
    __syncthreads();
    if constexpr (kFixedRef) decide(SA, 2 * j);
    const bool second = j * KT + KU < klen;
    if (second) qk(SB, 2 * j + 1);
    expv(SA, j, 0);
    if (second) {
      decide(SB, 2 * j + 1);
      expv(SB, j, 2);
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
    const int q = q0 + wave * QPW + qb * 32 + l32;
    if (q >= len) continue;
    if (splits > 1) {
      const int64_t pr = ((int64_t)split * part_rows + s0 + q) * n_heads + h;
      float* orow = opart + pr * HW;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * lhi;
          if (d >= HW) continue;
          *reinterpret_cast<float4*>(orow + d) = make_float4(
              O[db][qb][4 * g], O[db][qb][4 * g + 1], O[db][qb][4 * g + 2], O[db][qb][4 * g + 3]);
        }
      if (lhi == 0) lpart[pr] = lt;
      continue;
    }
    const float inv = 1.0f / lt;
    if (out_scale > 0.0f) {
      // E4M3 codes of the output times out_scale (the FP8 output projection's input)
      uint8_t* orow = reinterpret_cast<uint8_t*>(out) + (s0 + q) * hd + h * HW;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = db * 32 + 8 * g + 4 * lhi;
          const float sc = inv * out_scale;
          *reinterpret_cast<uint32_t*>(orow + d) =
              pack_fp8x4(O[db][qb][4 * g] * sc, O[db][qb][4 * g + 1] * sc,
                         O[db][qb][4 * g + 2] * sc, O[db][qb][4 * g + 3] * sc);
        }
      continue;
    }
    // rows of n_heads x HW; the last 32-dim block of a head narrower than a
    // multiple of 32 holds dims past HW, which are not stored
    bf16_t* orow = reinterpret_cast<bf16_t*>(out) + (s0 + q) * (int64_t)hd + h * HW;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db * 32 + 8 * g + 4 * lhi;
        if (d >= HW) continue;
        *reinterpret_cast<uint2*>(orow + d) =
            make_uint2(pack_bf16x2(O[db][qb][4 * g] * inv, O[db][qb][4 * g + 1] * inv),
                       pack_bf16x2(O[db][qb][4 * g + 2] * inv, O[db][qb][4 * g + 3] * inv));
      }
  }
}

// Output of a key-split launch: for every query row and head, the partial
// sums of the runs added in run order, O / l, stored as the unsplit kernel
// stores it (bf16).  One thread per 4 dims of a query row and head (every run's
// loads issued before the first add); blockIdx.y = head * n_tiles + tile.
constexpr int MAX_SPLITS = 8;
template <int HW>
__global__ __launch_bounds__(256) void attention_combine_kernel(
    const int4* __restrict__ tile_info, int n_tiles, int splits,
    const float* __restrict__ opart, const float* __restrict__ lpart, int64_t part_rows,
    bf16_t* __restrict__ out, int hd) {
  constexpr int V4 = HW / 4;   // 4-dim groups of a head row
  const int h = blockIdx.y / n_tiles;
  const int tile = blockIdx.y - h * n_tiles;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= QTILE * V4) return;
  const int4 ti = tile_info[tile];
  const int r = e / V4, c = e - r * V4;
  const int q = ti.z + r;
  if (q >= ti.y) return;
  const int64_t row = ti.x + q;
  const int n_heads = hd / HW;
  float4 t[MAX_SPLITS];
  float lv[MAX_SPLITS];
#pragma unroll
  for (int sp = 0; sp < MAX_SPLITS; ++sp) {
    if (sp < splits) {
      const int64_t pr = ((int64_t)sp * part_rows + row) * n_heads + h;
      t[sp] = *reinterpret_cast<const float4*>(opart + pr * HW + 4 * c);
      lv[sp] = lpart[pr];
    }
  }
  float4 o = t[0];
  float l = lv[0];
#pragma unroll
  for (int sp = 1; sp < MAX_SPLITS; ++sp) {
    if (sp < splits) {
      o.x += t[sp].x; o.y += t[sp].y; o.z += t[sp].z; o.w += t[sp].w;
      l += lv[sp];
    }
  }
  const float inv = 1.0f / l;
  *reinterpret_cast<uint2*>(out + row * hd + h * HW + 4 * c) =
      make_uint2(pack_bf16x2(o.x * inv, o.y * inv), pack_bf16x2(o.z * inv, o.w * inv));
}

}  // namespace

bool attention_fixed_ref_ok(const float* q_g, const float* q_b, const float* k_g,
                            const float* k_b, int dh) {
  // Norm bound of a head vector after LayerNorm (sum of squares of the
  // normalised values <= 128) with gain g and bias b, rotated (norm kept).
  auto norm_bound = [dh](const float* g, const float* b) {
    double gmax = 0.0, bsq = 0.0;
    for (int i = 0; i < dh; ++i) {
      gmax = std::max(gmax, std::fabs((double)g[i]));
      bsq += (double)b[i] * b[i];
    }
    return gmax * std::sqrt((double)dh) + std::sqrt(bsq);
  };
  // 2^-6 covers bf16 rounding of q and k and fp32 rounding of the products.
  const double bound = norm_bound(q_g, q_b) * norm_bound(k_g, k_b) * (1.0 + 1.0 / 64);
  const double log2_range = bound * 1.4426950408889634 / std::sqrt((double)dh);
  return std::isfinite(log2_range) && log2_range <= 64.0;
}

hipError_t launch_attention(const bf16_t* qkv, const int32_t* tile_info, int n_tiles,
                            int n_heads, int head_dim, bool fixed_ref, void* out, float out_scale,
                            int max_len, int64_t rows, float* opart, size_t opart_bytes,
                            float* lpart, size_t lpart_bytes, hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  if (n_heads < 1 || (head_dim != DH && head_dim != 80) || (out_scale > 0.0f && head_dim != DH))
    return hipErrorInvalidValue;
  const int n_items = n_tiles * n_heads;
  const int hd = n_heads * head_dim;
  // Key runs.  Two workgroups of this kernel fit a CU, so the work items run
  // in waves of 2 x CUs; for long sequences a launch whose items fill one
  // wave and a small part of the next (a 10-minute recording: 590 items for
  // 512 slots) pays a second full item time for that part.  Cutting each
  // item's keys into `splits` runs and adding the runs' partial sums in a
  // second pass shortens the items; the cut is taken when the modelled time
  // (waves x key tiles per run, plus the partial sums written and read back
  // at the cost of about one key tile per 8 MB) drops by a tenth.  Only long
  // sequences (the fixed costs of a workgroup are measured to dominate short
  // ones) and only with a fixed softmax reference, where runs add directly,
  // and a bf16 output (the E4M3 output of the FP8 variant keeps whole items).
  int splits = 1, t_split = 0;
  const int max_kt = (max_len + KT - 1) / KT;
  if (fixed_ref && out_scale <= 0.0f && opart && lpart && max_kt >= 32) {
    const int64_t slots = 2 * (int64_t)num_cus();
    auto waves = [&](int64_t units) { return (units + slots - 1) / slots; };
    const double base = (double)waves(n_items) * max_kt;
    double best = base;
    for (int sp = 2; sp <= MAX_SPLITS; ++sp) {
      const size_t obytes = (size_t)sp * rows * n_heads * head_dim * sizeof(float);
      const size_t lbytes = (size_t)sp * rows * n_heads * sizeof(float);
      if (obytes > opart_bytes || lbytes > lpart_bytes) break;
      const int per = (max_kt + sp - 1) / sp;
      const double cost = (double)waves((int64_t)n_items * sp) * per + 2.0 * obytes / 8e6;
      if (cost < best) {
        best = cost;
        splits = sp;
        t_split = per;
      }
    }
    if (best > 0.9 * base) splits = 1;
  }
  const int launch_items = n_items * splits;
  const int grid = (launch_items + 7) / 8 * 8;
  auto kernel = head_dim == DH
                    ? (fixed_ref ? attention_kernel<true, DH> : attention_kernel<false, DH>)
                    : (fixed_ref ? attention_kernel<true, 80> : attention_kernel<false, 80>);
  kernel<<<dim3(grid), dim3(64 * NW), 0, stream>>>(
      qkv, reinterpret_cast<const int4*>(tile_info), n_tiles, launch_items, out, out_scale, hd,
      splits, t_split, opart, lpart, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  auto combine = head_dim == DH ? attention_combine_kernel<DH> : attention_combine_kernel<80>;
  combine<<<dim3((QTILE * (head_dim / 4) + 255) / 256, n_items), dim3(256), 0, stream>>>(
      reinterpret_cast<const int4*>(tile_info), n_tiles, splits, opart, lpart, rows,
      reinterpret_cast<bf16_t*>(out), hd);
  return hipGetLastError();
}

}  // namespace enc
