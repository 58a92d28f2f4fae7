// bf16 MFMA GEMM for gfx950 with fused epilogues:
//   C[M, N] (op)= A[M, K] * W[N, K]^T + bias
// A holds activations (rows = packed positions), W a weight matrix in the
// [out, in] layout, both K-contiguous, fp32 accumulation.
//
// Used for the input projection (width 1024 -> 1280), the fused QKV
// projection, the attention output projection and the two FFN matrices of
// "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
// "How audio and speakers reach the language model" (width 1,280, feed-forward
// expansion four; the activation is not named there, and exact-erf GELU is the
// reading taken).
//
// Two kernels share the output tiling (256 x 256 tiles, numbered in groups of
// four tile rows so that neighbouring tiles share A rows and W columns):
//
//  * gemm_big_kernel -- persistent, one workgroup per CU, eight wavefronts
//    of 128 x 64 outputs each in two groups that alternate between running
//    MFMAs and issuing loads / storing results (see its own comment).  It
//    covers every full round of tiles.  Operands go straight from global
//    memory into LDS with global_load_lds_dwordx4 (no register staging; the
//    XOR swizzle that keeps the MFMA operand reads conflict-free is applied on
//    the global side by choosing which 16-byte chunk each lane fetches), in
//    64-wide K slices of whole 128-byte lines.  The stream of steps runs on
//    across the workgroup's tiles.
//  * gemm_small_kernel (+ gemm_small_reduce) -- the tiles left after the
//    last full round, as 64 x 64 pieces, and the whole product when it has
//    fewer 256 x 256 tiles than CUs (few rows), as 64 x 64 or 128 x 64
//    pieces, split along K only when even these leave CUs idle.
//
// Each lane ends up owning one output row and runs of four consecutive
// columns: the epilogue adds bias / residual / GELU in registers and stores
// 8- or 16-byte vectors.

#include <algorithm>
#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr int BIG = 256;    // big tile edge
constexpr int GROUP_M = 4;  // tile rows per ordering group

// Exact-erf GELU, x Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), with erf taken from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erf(z) = 1 - P(t) exp(-z^2), P(t) = a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5,
// t = 1 / (1 + p z), z >= 0, absolute error below 1.5e-7 -- far below the
// bf16 rounding of the output.  With z = |x| / sqrt 2 both signs of x give
// x Phi(x) = max(x, 0) - 0.5 |x| P(t) exp(-x^2 / 2), which takes one
// reciprocal, one exponential (exp2 of -x^2 log2(e) / 2) and eleven other
// operations (the 0.5 is folded into the coefficients).
__device__ __forceinline__ float gelu_erf(float x) {
  const float a = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, a, 1.0f));
  float p = fmaf(0.5f * 1.061405429f, t, 0.5f * -1.453152027f);
  p = fmaf(p, t, 0.5f * 1.421413741f);
  p = fmaf(p, t, 0.5f * -0.284496736f);
  p = fmaf(p, t, 0.5f * 0.254829592f);
  const float e = __builtin_amdgcn_exp2f(x * (x * -0.72134752044448170f));
  return fmaf(-(a * t) * p, e, x > 0.0f ? x : 0.0f);
}

// Big-tile coordinates of tile t: groups of GROUP_M tile rows, column-major
// inside a group, so that consecutive tiles (which run together on one XCD)
// touch few distinct A row blocks and W column blocks.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GROUP_M * tiles_n;
  const int group = t / per_group;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int r = t - group * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// Apply the epilogue to four consecutive columns n..n+3 of row m; bv holds
// their biases.
// The FP8 path first multiplies the accumulators by alpha (the product of the
// two operand scales); kBiasGeluFp8 scales its result by oscale and stores
// E4M3 codes (ldc in bytes).
template <Epilogue EPI, bool F8>
__device__ __forceinline__ void store4(void* __restrict__ Cv, int64_t ldc, int64_t m, int n,
                                       float4 bv, float alpha, float oscale, float a0, float a1,
                                       float a2, float a3) {
  if constexpr (F8) {
    a0 *= alpha; a1 *= alpha; a2 *= alpha; a3 *= alpha;
  }
  float o0 = a0 + bv.x, o1 = a1 + bv.y, o2 = a2 + bv.z, o3 = a3 + bv.w;
  if constexpr (EPI == Epilogue::kBiasGeluBf16 || EPI == Epilogue::kBiasGeluFp8) {
    o0 = gelu_erf(o0); o1 = gelu_erf(o1); o2 = gelu_erf(o2); o3 = gelu_erf(o3);
  }
  if constexpr (EPI == Epilogue::kBiasGeluFp8) {
    uint8_t* C = reinterpret_cast<uint8_t*>(Cv);
    *reinterpret_cast<uint32_t*>(C + m * ldc + n) =
        pack_fp8x4(o0 * oscale, o1 * oscale, o2 * oscale, o3 * oscale);
  } else if constexpr (EPI == Epilogue::kBiasBf16 || EPI == Epilogue::kBiasGeluBf16) {
    bf16_t* C = reinterpret_cast<bf16_t*>(Cv);
    *reinterpret_cast<uint2*>(C + m * ldc + n) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
  } else {
    float* C = reinterpret_cast<float*>(Cv);
    float4* dst = reinterpret_cast<float4*>(C + m * ldc + n);
    if constexpr (EPI == Epilogue::kBiasResidualF32) {
      const float4 r = *dst;
      o0 += r.x; o1 += r.y; o2 += r.z; o3 += r.w;
    }
    *dst = make_float4(o0, o1, o2, o3);
  }
}

// Biases of columns nb + 8q + 4 lhi .. +3 for q = 0..3.  nb is uniform across
// the wavefront, so the 32 values come through scalar loads (which do not
// queue behind the vector-memory DMAs still in flight); each lane then keeps
// the half that matches its lhi.
__device__ __forceinline__ void load_bias32(const float* __restrict__ bias, int nb, int lhi,
                                            float4 (&bv)[4]) {
  nb = __builtin_amdgcn_readfirstlane(nb);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 lo = *reinterpret_cast<const float4*>(bias + nb + 8 * q);
    const float4 hi = *reinterpret_cast<const float4*>(bias + nb + 8 * q + 4);
    bv[q] = lhi ? hi : lo;
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte-per-lane DMA from global memory into LDS (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds + 16 l.
__device__ __forceinline__ void dma16(const void* gptr, lds_void* lds) {
  __builtin_amdgcn_global_load_lds(gptr, lds, 16, 0, 0);
}

// ------------------------------------------------- big (persistent, 8 waves)
// 256 x 256 tiles in 64-wide K steps.  Eight wavefronts in two groups of
// four, one wavefront of each group per SIMD; group g owns output rows
// 128 g .. 128 g + 127 of the tile and wave q of a group the columns
// 64 q .. 64 q + 63 (eight 32x32 accumulators, 128 registers).  A slices
// (256 rows x 64 K, 32 KB) rotate through three LDS slots and W slices
// through two (160 KB).  Each step has two phases separated by a barrier:
//   phase 1: group 0 runs its MFMAs on step g; group 1 sends the direct loads
//            of W for step g+1 (and, at a tile's first step, stores its part
//            of the previous tile);
//   phase 2: group 1 runs its MFMAs on step g; group 0 sends the loads of A
//            for step g+2 (and, at a tile's last step, stores its part).
// A wavefront that is issuing loads (which can stall for hundreds of cycles
// when the load path is busy) or storing results is never the one feeding
// the matrix cores of its SIMD, and the stores of one tile spread over two
// phases instead of leaving every CU idle at once.
// In bf16 each group reads a step's first operand fragments from LDS at the
// start of its own compute phase and covers their latency with the MFMAs of
// the previous step's last 16-wide k, which it held back (see compute0).
// Direct load of 16 bytes per lane from sbase + voff to LDS byte address
// lds + 16 * lane (sbase and lds uniform).  Written in asm so that the
// compiler does not track it: the kernel waits for these loads explicitly
// (wait_vm0) before the barrier that publishes a slot, and the compiler would
// otherwise stall every LDS read it cannot prove disjoint from a slot in
// flight.  M0 is not used otherwise by this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_s(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// LDS reads issued by this wavefront have completed (before a barrier after
// which another wavefront, or this one, may refill the slot they read).
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int PBK = 64;   // K step of the persistent kernel

// F8: A and W hold E4M3 codes and every length along K (K, lda, ldw) is given
// in units of two codes, so the data movement below is the bf16 one byte for
// byte; one 64-code MFMA step takes the two consecutive 16-byte fragments a
// lane would feed to two bf16 steps (A and W use the same assignment of
// bytes to k, so every product pairs the right codes).
template <Epilogue EPI, bool F8, bool XA>
__global__ __launch_bounds__(512, 1) void gemm_big_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ bias, void* __restrict__ Cv, int64_t ldc, int64_t M, int K,
    int tiles_m, int tiles_n, int n_big, float alpha, float oscale) {
  constexpr int SL = BIG * PBK / 8;   // uint4 per slot (32 KB)
  __shared__ uint4 sA[3][SL];
  __shared__ uint4 sW[2][SL];

  const int G = gridDim.x;
  const int wg = blockIdx.x;
  const int slot = (G % 8 == 0) ? (wg % 8) * (G / 8) + wg / 8 : wg;
  const int my_tiles = slot < n_big ? (n_big - 1 - slot) / G + 1 : 0;
  const int KT = K / PBK;
  const int total = my_tiles * KT;
  // XA: residual tile preloaded into the accumulators (see below the epilogue)
  static_assert(!XA || (EPI == Epilogue::kBiasResidualF32 && !F8), "XA: bf16 residual products");
  constexpr bool x_in_acc = XA;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int q = wave & 3;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // Piece t of a slice = rows 8t .. 8t+7; wave q of the loading group fills
  // pieces 8q .. 8q+7; lane -> row 8t + lane/8, LDS chunk lane%8 of the row
  // holds global chunk (lane%8) ^ ((row/2)%8).  Rows past M (last row tile
  // only) re-read row M-1.
  //   bf16: the eight per-lane offsets are kept in registers (recomputed when
  //         the A tile changes).
  //   FP8 and the bf16-output epilogue (whose lane exchanges need the
  //         registers): offsets computed per call: with
  //         row = 64q + 8t' + lane/8 (t' = t - 8q) the swizzle depends only on
  //         the parity of t' and on lane/16, so two offsets are computed per
  //         call and the 8t'-row step goes into the uniform base address.
  const uint32_t ldsA = (uint32_t)(uintptr_t)(lds_void*)&sA[0][0];
  const uint32_t ldsW = (uint32_t)(uintptr_t)(lds_void*)&sW[0][0];
  uint32_t off[8];
  int off_tile = -1;
  auto issue = [&](int g, bool is_a) __attribute__((always_inline)) {
    const int r = g / KT, kt = g - r * KT;
    int tm, tn;
    tile_coords(r * G + slot, tiles_m, tiles_n, tm, tn);
    const int64_t am = (int64_t)tm * BIG;
    if constexpr (!F8 && EPI != Epilogue::kBiasBf16 && !XA) {
      if (is_a) {
        if (off_tile != r) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int rr = (q * 8 + t) * 8 + (lane >> 3);
            const int c = ((lane & 7) ^ ((rr >> 1) & 7)) * 8;
            const int64_t row = min<int64_t>(am + rr, M - 1) - am;
            off[t] = (uint32_t)((row * lda + c) * 2);
          }
          off_tile = r;
        }
        const char* base = reinterpret_cast<const char*>(A + am * lda) + kt * PBK * 2;
        const uint32_t l = ldsA + (g % 3) * (SL * 16) + q * 8 * 1024;
#pragma unroll
        for (int t = 0; t < 8; ++t) dma16_s(base, off[t], l + t * 1024);
      } else {
        if (off_tile != -2) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int rr = (q * 8 + t) * 8 + (lane >> 3);
            const int c = ((lane & 7) ^ ((rr >> 1) & 7)) * 8;
            off[t] = (uint32_t)((rr * ldw + c) * 2);
          }
          off_tile = -2;
        }
        const char* base =
            reinterpret_cast<const char*>(W + (int64_t)tn * BIG * ldw) + kt * PBK * 2;
        const uint32_t l = ldsW + (g & 1) * (SL * 16) + q * 8 * 1024;
#pragma unroll
        for (int t = 0; t < 8; ++t) dma16_s(base, off[t], l + t * 1024);
      }
      return;
    }
    // FP8 (the empty asm keeps the offsets from being hoisted out of the loop,
    // where they would be spilled and reloaded through memory)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int rl = q * 64 + (ln >> 3);
    const int sw = ln >> 4;
    const int ce = ((ln & 7) ^ sw) * 8;
    const int co = ((ln & 7) ^ (sw + 4)) * 8;
    if (is_a) {
      const char* base = reinterpret_cast<const char*>(A + am * lda) + kt * PBK * 2;
      const uint32_t l = ldsA + (g % 3) * (SL * 16) + q * 8 * 1024;
      if (am + BIG <= M) {
        const uint32_t ve = (uint32_t)((rl * lda + ce) * 2);
        const uint32_t vo = (uint32_t)((rl * lda + co) * 2);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          dma16_s(base + (int64_t)t * 16 * lda, (t & 1) ? vo : ve, l + t * 1024);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t row = min<int64_t>(am + rl + 8 * t, M - 1) - am;
          dma16_s(base, (uint32_t)((row * lda + ((t & 1) ? co : ce)) * 2), l + t * 1024);
        }
      }
    } else {
      const char* base =
          reinterpret_cast<const char*>(W + (int64_t)tn * BIG * ldw) + kt * PBK * 2;
      const uint32_t l = ldsW + (g & 1) * (SL * 16) + q * 8 * 1024;
      const uint32_t ve = (uint32_t)((rl * ldw + ce) * 2);
      const uint32_t vo = (uint32_t)((rl * ldw + co) * 2);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        dma16_s(base + (int64_t)t * 16 * ldw, (t & 1) ? vo : ve, l + t * 1024);
    }
  };

  const int rsw = (l32 >> 1) & 7;
  const int aofs = (grp * 128 + l32) * 8;
  const int wofs = (q * 64 + l32) * 8;

  f32x16 acc[2][4];
  bf16x8 f0[6], f1[6];
  auto load = [&](const uint4* a, const uint4* w, int sl, bf16x8 (&f)[6])
      __attribute__((always_inline)) {
    // in the order the MFMAs consume them (W 0 and A 0 feed the first)
    const int pc = (2 * sl + lhi) ^ rsw;
    f[0] = __builtin_bit_cast(bf16x8, w[wofs + pc]);
    f[2] = __builtin_bit_cast(bf16x8, a[aofs + pc]);
    f[1] = __builtin_bit_cast(bf16x8, w[wofs + 256 + pc]);
#pragma unroll
    for (int j = 1; j < 4; ++j) f[2 + j] = __builtin_bit_cast(bf16x8, a[aofs + j * 256 + pc]);
  };
  auto mma = [&](const bf16x8 (&f)[6], bool fresh) __attribute__((always_inline)) {
    const f32x16 z = {};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[i], f[2 + j], fresh ? z : acc[i][j],
                                                            0, 0, 0);
  };
  auto interleave = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 6; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  };
  auto compute = [&](const uint4* a, const uint4* w, bool first) __attribute__((always_inline)) {
    load(a, w, 1, f1);
    mma(f0, first);
    interleave();
    load(a, w, 2, f0);
    mma(f1, false);
    interleave();
    load(a, w, 3, f1);
    mma(f0, false);
    interleave();
    mma(f1, false);
  };
  // bf16: a group reads its first fragments of a step at the start of its
  // compute phase (group 0 could not read them earlier: the barrier that
  // opens its phase publishes them).  It holds back the MFMAs of a step's
  // last 16-wide k (their fragments stay in f1) and issues them at the start
  // of its next compute phase, where they cover the latency of those reads.
  // The order of summation is unchanged; a tile's last step completes in
  // full, so nothing is held across an epilogue.
  auto compute0 = [&](const uint4* a, const uint4* w, bool first, bool pending, bool defer)
      __attribute__((always_inline)) {
    load(a, w, 0, f0);
    if (pending) {
      mma(f1, false);
      interleave();
    }
    load(a, w, 1, f1);
    mma(f0, first);
    interleave();
    load(a, w, 2, f0);
    mma(f1, false);
    interleave();
    load(a, w, 3, f1);
    mma(f0, false);
    interleave();
    if (!defer) mma(f1, false);
  };
  // FP8: code step ks covers bf16 steps 2 ks and 2 ks + 1; a fragment is the
  // two 16-byte chunks of those steps.  Step 1's fragments are read while
  // step 0's MFMAs run, each A fragment only after the two MFMAs that use
  // the previous one, so that at most one step plus two fragments are live.
  auto ld8 = [&](const uint4* base, int ofs, int ks) __attribute__((always_inline)) {
    const i32x4 lo = __builtin_bit_cast(i32x4, base[ofs + ((4 * ks + lhi) ^ rsw)]);
    const i32x4 hi = __builtin_bit_cast(i32x4, base[ofs + ((4 * ks + 2 + lhi) ^ rsw)]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  i32x8 gw0, gw1, ga[4];
  auto mma8 = [&](const i32x8& w0, const i32x8& w1, const i32x8& aj, int j, bool fresh)
      __attribute__((always_inline)) {
    const f32x16 z = {};
    acc[0][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w0, aj, fresh ? z : acc[0][j], 0,
                                                                0, 0, 0, 0, 0);
    acc[1][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w1, aj, fresh ? z : acc[1][j], 0,
                                                                0, 0, 0, 0, 0);
  };
  auto compute8 = [&](const uint4* a, const uint4* w, bool first) __attribute__((always_inline)) {
    const i32x8 nw0 = ld8(w, wofs, 1);
    const i32x8 nw1 = ld8(w, wofs + 256, 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mma8(gw0, gw1, ga[j], j, first);
      ga[j] = ld8(a, aofs + j * 256, 1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) mma8(nw0, nw1, ga[j], j, false);
    // order: next W reads; per A fragment two MFMAs then its replacement's
    // reads; then the second step's eight MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };
  auto preload = [&](const uint4* a, const uint4* w) __attribute__((always_inline)) {
    if constexpr (F8) {
      gw0 = ld8(w, wofs, 0);
      gw1 = ld8(w, wofs + 256, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) ga[j] = ld8(a, aofs + j * 256, 0);
    } else {
      load(a, w, 0, f0);
    }
  };
  auto step = [&](const uint4* a, const uint4* w, bool first) __attribute__((always_inline)) {
    if constexpr (F8) compute8(a, w, first);
    else compute(a, w, first);
  };
  auto epilogue = [&](int r) __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(r * G + slot, tiles_m, tiles_n, tm, tn);
    const int64_t mb = (int64_t)tm * BIG + grp * 128 + l32;
    const int nw = tn * BIG + q * 64;
    // (measured: the bf16 GELU output, which also needs its load offsets
    // cached for registers' sake, is faster with the plain stores below)
    if constexpr (EPI == Epilogue::kBiasBf16 || EPI == Epilogue::kBiasGeluFp8) {
      // Narrow outputs: lanes l and l + 32 hold the same row, columns
      // 8 qq + 0..3 and 8 qq + 4..7.  Exchanging the packed chunks of qq = 2p
      // and 2p + 1 between the two halves (v_permlane32_swap) leaves each lane
      // 8 consecutive columns, so half as many, twice as wide stores.
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float4 bv[4];
        load_bias32(bias, nw + i * 32, lhi, bv);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = mb + j * 32;
          uint32_t pk[4][2];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = acc[i][j][4 * qq + e];
              if constexpr (F8) v *= alpha;
              o[e] = v + (e == 0 ? bv[qq].x : e == 1 ? bv[qq].y : e == 2 ? bv[qq].z : bv[qq].w);
              if constexpr (EPI != Epilogue::kBiasBf16) o[e] = gelu_erf(o[e]);
            }
            if constexpr (EPI == Epilogue::kBiasGeluFp8) {
              pk[qq][0] = pack_fp8x4(o[0] * oscale, o[1] * oscale, o[2] * oscale, o[3] * oscale);
              pk[qq][1] = 0;
            } else {
              pk[qq][0] = pack_bf16x2(o[0], o[1]);
              pk[qq][1] = pack_bf16x2(o[2], o[3]);
            }
          }
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int n = nw + i * 32 + 16 * p + 8 * lhi;
            const auto s0 = __builtin_amdgcn_permlane32_swap(pk[2 * p][0], pk[2 * p + 1][0],
                                                             false, false);
            if constexpr (EPI == Epilogue::kBiasGeluFp8) {
              if (m < M)
                *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(Cv) + m * ldc + n) =
                    make_uint2(s0[0], s0[1]);
            } else {
              const auto s1 = __builtin_amdgcn_permlane32_swap(pk[2 * p][1], pk[2 * p + 1][1],
                                                               false, false);
              if (m < M)
                *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(Cv) + m * ldc + n) =
                    make_uint4(s0[0], s1[0], s0[1], s1[1]);
            }
          }
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float4 bv[4];
      load_bias32(bias, nw + i * 32, lhi, bv);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = mb + j * 32;
        if (m < M) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            if constexpr (x_in_acc)   // the residual is already in the accumulators
              store4<Epilogue::kBiasF32, F8>(Cv, ldc, m, nw + i * 32 + 8 * qq + 4 * lhi, bv[qq],
                                             alpha, oscale, acc[i][j][4 * qq],
                                             acc[i][j][4 * qq + 1], acc[i][j][4 * qq + 2],
                                             acc[i][j][4 * qq + 3]);
            else
              store4<EPI, F8>(Cv, ldc, m, nw + i * 32 + 8 * qq + 4 * lhi, bv[qq], alpha, oscale,
                              acc[i][j][4 * qq], acc[i][j][4 * qq + 1], acc[i][j][4 * qq + 2],
                              acc[i][j][4 * qq + 3]);
          }
        }
      }
    }
  };

  // XA (residual products whose tiles make exactly one round, e.g. the
  // attention output and FFN-down projections of a batch of ~13k rows): the
  // tile's fp32 residual is loaded into the accumulators before the first
  // MFMA, under the pipeline fill, instead of being read back in the
  // epilogue, where every CU would read it at the same moment; the epilogue
  // then adds the bias and stores.  (The sum x + (products) + bias is formed
  // in that order instead of x + (products + bias).)
  auto load_x = [&]() __attribute__((always_inline)) {
    int tm, tn;
    tile_coords(slot, tiles_m, tiles_n, tm, tn);
    const int64_t mb = (int64_t)tm * BIG + grp * 128 + l32;
    const int nw = tn * BIG + q * 64;
    const float* X = reinterpret_cast<const float*>(Cv);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = min<int64_t>(mb + 32 * j, M - 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float4 v =
              *reinterpret_cast<const float4*>(X + m * ldc + nw + 32 * i + 8 * qq + 4 * lhi);
          acc[i][j][4 * qq] = v.x;
          acc[i][j][4 * qq + 1] = v.y;
          acc[i][j][4 * qq + 2] = v.z;
          acc[i][j][4 * qq + 3] = v.w;
        }
    }
  };
  // Prologue: A of steps 0 and 1 (group 0), W of step 0 (group 1).
  if (total > 0) {
    if (grp == 0) {
      issue(0, true);
      if (total > 1) issue(1, true);
      wait_vm0();
    } else {
      issue(0, false);
      wait_vm0();
    }
  }
  wg_barrier();
  if constexpr (!F8) {
    // bf16: each group runs a loop of its own, so that its held-back
    // fragments (compute0) are live only where it needs them.  Both loops
    // pass two barriers per step.  Each peels a tile's first step (no
    // held-back MFMAs to issue; group 1 stores the previous tile there) and
    // last step (none to hold back; group 0 stores the tile there) out of its
    // inner loop, so held-back fragments are never live across an epilogue.
    if (grp == 0) {
      auto phase2 = [&](int g) __attribute__((always_inline)) {
        wg_barrier();
        wait_vm0();   // A(g+1), issued a step ago
        if (g + 2 < total) issue(g + 2, true);   // into the slot of A(g-1)
        // the held-back fragments' reads of A(g) and W(g), issued a phase
        // ago, have completed before the barrier after which group 1 writes
        // W(g+2) over W(g)
        wait_lgkm0();
      };
#pragma unroll 1
      for (int r = 0; r < my_tiles; ++r) {
        const int g0 = r * KT;
        if constexpr (x_in_acc) load_x();   // the only tile
        compute0(sA[g0 % 3], sW[g0 & 1], !x_in_acc, false, true);
        phase2(g0);
        wg_barrier();
#pragma unroll 1
        for (int kt = 1; kt < KT - 1; ++kt) {
          const int g = g0 + kt;
          compute0(sA[g % 3], sW[g & 1], false, true, true);
          phase2(g);
          wg_barrier();
        }
        const int gl = g0 + KT - 1;
        compute0(sA[gl % 3], sW[gl & 1], false, true, false);
        phase2(gl);
        epilogue(r);
        wg_barrier();
      }
    } else {
      auto phase1 = [&](int g) __attribute__((always_inline)) {
        // the held-back fragments' reads of A(g-1) and W(g-1), issued a phase
        // ago, have completed before W(g+1) is written over W(g-1) and before
        // the barrier after which group 0 writes A(g+2) over A(g-1)
        wait_lgkm0();
        if (g + 1 < total) issue(g + 1, false);   // W(g+1) into the slot of W(g-1)
      };
      auto phase2 = [&](int g, bool first, bool pending, bool defer)
          __attribute__((always_inline)) {
        wg_barrier();
        compute0(sA[g % 3], sW[g & 1], first, pending, defer);
        wait_vm0();   // W(g+1) landed
        wg_barrier();
      };
#pragma unroll 1
      for (int r = 0; r < my_tiles; ++r) {
        const int g0 = r * KT;
        phase1(g0);
        if (r > 0) epilogue(r - 1);
        if constexpr (x_in_acc) load_x();   // the only tile, under group 0's first phase
        phase2(g0, !x_in_acc, false, true);
#pragma unroll 1
        for (int kt = 1; kt < KT - 1; ++kt) {
          phase1(g0 + kt);
          phase2(g0 + kt, false, true, true);
        }
        phase1(g0 + KT - 1);
        phase2(g0 + KT - 1, false, true, false);
      }
      if (total > 0) epilogue(my_tiles - 1);
    }
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  for (int g = 0; g < total; ++g) {
    const int r = g / KT, kt = g - r * KT;
    const uint4* a = sA[g % 3];
    const uint4* w = sW[g & 1];
    // phase 1: group 0 computes, group 1 loads W(g+1)
    if (grp == 0) {
      preload(a, w);
      if (kt == 0) step(a, w, true);
      else step(a, w, false);
    } else {
      if (g + 1 < total) issue(g + 1, false);
      if (kt == 0 && r > 0) epilogue(r - 1);
      preload(a, w);
    }
    wg_barrier();
    // phase 2: group 1 computes, group 0 loads A(g+2)
    if (grp == 1) {
      if (kt == 0) step(a, w, true);
      else step(a, w, false);
      wait_vm0();   // W(g+1) landed
    } else {
      // A(g+1), issued a step ago, must have landed before the barrier; wait
      // for it first, so that no count of younger operations is needed.
      wait_vm0();
      if (g + 2 < total) issue(g + 2, true);
      if (kt == KT - 1) epilogue(r);
    }
    wg_barrier();
  }
  if (grp == 1 && total > 0) epilogue(my_tiles - 1);
  __builtin_amdgcn_s_waitcnt(0);
}

// ------------------------------------------------- pieces (few rows, tails)
// Whole products with fewer 256 x 256 tiles than CUs (a 30-second clip: 375
// rows) are cut into 64 x 64 (or 128 x 64, see launch_t) pieces.  That gives every CU work without
// splitting K for most shapes, so no partial sums are written and no
// reduction runs.  A workgroup of four wavefronts (32 x 32 outputs each, one
// accumulator) moves 64-wide K slices of A and W (whole 128-byte lines) into
// a ring of four 16 KB LDS stages by direct loads, three in flight; the
// kernel is bound by that data movement, not by its MFMAs.  Products that
// still leave CUs idle split K, with partial sums and gemm_small_reduce.
constexpr int SP = 64;    // piece edge
constexpr int SBK = 64;   // K step
constexpr int SNS = 4;    // ring stages

// Piece pid's first row and column: mode 0, the sixteen 64 x 64 pieces of
// each big tile t_begin, t_begin + 1, ...; mode 1, a plain grid of pieces_n
// pieces of PM rows x 64 columns per piece row.
struct SmallMap {
  int mode;
  int t_begin, tiles_m, tiles_n;   // mode 0
  int pieces_n;                    // mode 1
};

template <int PM>
__device__ __forceinline__ void small_coords(int pid, const SmallMap& sm, int64_t& m0,
                                             int64_t& n0) {
  if (PM == SP && sm.mode == 0) {
    int tm, tn;
    tile_coords(sm.t_begin + (pid >> 4), sm.tiles_m, sm.tiles_n, tm, tn);
    m0 = (int64_t)tm * BIG + (pid & 3) * SP;
    n0 = (int64_t)tn * BIG + ((pid >> 2) & 3) * SP;
  } else {
    m0 = (int64_t)(pid / sm.pieces_n) * PM;
    n0 = (int64_t)(pid % sm.pieces_n) * SP;
  }
}

// PM: rows of a piece, 64 (two workgroups per CU) or 128 (each wavefront
// 64 x 32 outputs in two accumulators; a 24 KB stage moves 128 + 64 rows for
// twice the products of a 64 x 64 piece, 43 instead of 32 flops per byte).
// F8: E4M3 codes moved as pairs (K, lda, ldw in units of two codes), as in
// the other kernels; a 64-code MFMA takes the fragments of two bf16 k-steps.
template <Epilogue EPI, bool PARTIAL, bool F8, int PM>
__global__ __launch_bounds__(256, PM == SP ? 2 : 1) void gemm_small_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ bias, void* __restrict__ Cv, int64_t ldc, float* __restrict__ part,
    int64_t M, int K, SmallMap sm, int splits, float alpha, float oscale) {
  static_assert(PM == SP || PM == 2 * SP, "piece rows");
  constexpr int NB = (PM + SP) / 8;        // 8-row blocks of a stage: A rows, then W rows
  constexpr int NBW = NB / 4;              // blocks per wavefront
  constexpr int NA = PM / SP;              // accumulators per wavefront
  constexpr int STG = NB * 64;             // uint4 per stage (16 or 24 KB)
  __shared__ uint4 st[SNS][STG];

  const int split = blockIdx.x % splits;
  const int pid = blockIdx.x / splits;
  int64_t m0, n0;
  small_coords<PM>(pid, sm, m0, n0);
  if (m0 >= M) return;   // a piece of the last tile row wholly past M
  const int kc = K / splits;
  const int kb = split * kc;
  const int KT = kc / SBK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // DMA: a stage is NB blocks of 8 rows x 128 bytes (A rows 0..PM-1, then W
  // rows 0..63); wave w fills blocks NBW w .. NBW w + NBW - 1, lane l the LDS
  // chunk l % 8 of row l / 8 of a block, which holds global chunk
  // (l % 8) ^ ((row / 2) % 8) (the XOR keeps the operand reads below
  // conflict-free).
  const bf16_t* src[NBW];
#pragma unroll
  for (int t = 0; t < NBW; ++t) {
    const int blk = wave * NBW + t;
    const bool is_a = blk < PM / 8;
    const int row = (is_a ? blk : blk - PM / 8) * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    src[t] = is_a ? A + min<int64_t>(m0 + row, M - 1) * lda + kb + chunk * 8
                  : W + (n0 + row) * ldw + kb + chunk * 8;
  }
  int ikt = 0;
  auto issue = [&](int slot) __attribute__((always_inline)) {
    const int k0 = min(ikt, KT - 1) * SBK;   // past the end: re-read the last step
#pragma unroll
    for (int t = 0; t < NBW; ++t)
      dma16(src[t] + k0, (lds_void*)(&st[slot][0] + (wave * NBW + t) * 64));
    ++ikt;
  };

  // operand rows: A rows wm*PM/2 + 32 b + l32, W row wn*32 + l32 (LDS rows of
  // 8 chunks)
  const int rsw = (l32 >> 1) & 7;
  const int aofs = (wm * (PM / 2) + l32) * 8;
  const int wofs = PM * 8 + (wn * 32 + l32) * 8;
  f32x16 acc[NA];
#pragma unroll
  for (int b = 0; b < NA; ++b)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[b][v] = 0.f;

  constexpr int VM = NBW * (SNS - 2);
  constexpr int WAIT_STEP = (VM & 15) | ((VM >> 4) << 14) | 0x0070;   // vmcnt(VM) lgkmcnt(0)
#pragma unroll
  for (int i = 0; i < SNS - 1; ++i) issue(i);
  for (int kt = 0; kt < KT; ++kt) {
    __builtin_amdgcn_s_waitcnt(WAIT_STEP);   // this step's stage has landed
    __builtin_amdgcn_s_barrier();            // ... for every wavefront; the oldest stage is free
    issue((kt + SNS - 1) % SNS);
    const uint4* sp = st[kt % SNS];
    bf16x8 fa[NA][4], fw[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const int pc = (2 * sl + lhi) ^ rsw;
      fw[sl] = __builtin_bit_cast(bf16x8, sp[wofs + pc]);
#pragma unroll
      for (int b = 0; b < NA; ++b)
        fa[b][sl] = __builtin_bit_cast(bf16x8, sp[aofs + b * 256 + pc]);
    }
    if constexpr (F8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int b = 0; b < NA; ++b)
          acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              __builtin_shufflevector(__builtin_bit_cast(i32x4, fw[2 * h]),
                                      __builtin_bit_cast(i32x4, fw[2 * h + 1]), 0, 1, 2, 3, 4, 5,
                                      6, 7),
              __builtin_shufflevector(__builtin_bit_cast(i32x4, fa[b][2 * h]),
                                      __builtin_bit_cast(i32x4, fa[b][2 * h + 1]), 0, 1, 2, 3, 4,
                                      5, 6, 7),
              acc[b], 0, 0, 0, 0, 0, 0);
    } else {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int b = 0; b < NA; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[sl], fa[b][sl], acc[b], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // loads past the last step land before LDS is released

  const int nw = (int)n0 + wn * 32;
  if constexpr (PARTIAL) {
    // partial layout: [pid][split][PM rows][64 cols] fp32
#pragma unroll
    for (int b = 0; b < NA; ++b) {
      float* dst = part + ((int64_t)pid * splits + split) * (PM * SP) +
                   (wm * (PM / 2) + 32 * b + l32) * SP + wn * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 8 * q + 4 * lhi) =
            make_float4(acc[b][4 * q], acc[b][4 * q + 1], acc[b][4 * q + 2], acc[b][4 * q + 3]);
    }
  } else {
    float4 bv[4];
    load_bias32(bias, nw, lhi, bv);
#pragma unroll
    for (int b = 0; b < NA; ++b) {
      const int64_t m = m0 + wm * (PM / 2) + 32 * b + l32;
      if (m < M) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          store4<EPI, F8>(Cv, ldc, m, nw + 8 * q + 4 * lhi, bv[q], alpha, oscale, acc[b][4 * q],
                          acc[b][4 * q + 1], acc[b][4 * q + 2], acc[b][4 * q + 3]);
      }
    }
  }
}

// Sum the split partials of each PM x 64 piece in split order and apply the
// epilogue; one thread per 4 consecutive columns.
template <Epilogue EPI, bool F8, int PM>
__global__ __launch_bounds__(256) void gemm_small_reduce(const float* __restrict__ part,
                                                         const float* __restrict__ bias,
                                                         void* __restrict__ Cv, int64_t ldc,
                                                         int64_t M, SmallMap sm, int splits,
                                                         float alpha, float oscale) {
  const int pid = blockIdx.y;
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;   // element in the piece
  int64_t m0, n0;
  small_coords<PM>(pid, sm, m0, n0);
  const int64_t m = m0 + e / SP;
  const int n = (int)n0 + e % SP;
  if (m >= M) return;
  const float* src = part + (int64_t)pid * splits * (PM * SP) + e;
  float4 s = *reinterpret_cast<const float4*>(src);
  for (int k = 1; k < splits; ++k) {
    const float4 t = *reinterpret_cast<const float4*>(src + (int64_t)k * (PM * SP));
    s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
  }
  store4<EPI, F8>(Cv, ldc, m, n, *reinterpret_cast<const float4*>(bias + n), alpha, oscale, s.x,
                  s.y, s.z, s.w);
}


// Split K (a divisor of K / 64) only while the pieces that hold rows still
// fit one workgroup per CU and their partial sums fit `part`.
// `live` pieces hold rows (of `pieces` launched).
int small_splits(int K, int live, int pieces, int pm, int cus, size_t part_bytes) {
  const int units = K / SBK;
  int splits = 1;
  for (int sp = 2; sp <= units; ++sp) {
    if (units % sp) continue;
    if ((int64_t)live * sp > cus) break;
    if ((size_t)pieces * sp * pm * SP * sizeof(float) > part_bytes) break;
    splits = sp;
  }
  return splits;
}

template <Epilogue EPI, bool F8, int PM>
hipError_t launch_small(const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw,
                        const float* bias, void* C, int64_t ldc, int64_t M, int K, float* part,
                        size_t part_bytes, const SmallMap& sm, int live, int pieces, int cus,
                        float alpha, float oscale, hipStream_t stream) {
  const int splits = small_splits(K, live, pieces, PM, cus, part_bytes);
  if (splits == 1) {
    gemm_small_kernel<EPI, false, F8, PM><<<dim3(pieces), dim3(256), 0, stream>>>(
        A, lda, W, ldw, bias, C, ldc, part, M, K, sm, 1, alpha, oscale);
    return hipGetLastError();
  }
  gemm_small_kernel<EPI, true, F8, PM><<<dim3(pieces * splits), dim3(256), 0, stream>>>(
      A, lda, W, ldw, bias, C, ldc, part, M, K, sm, splits, alpha, oscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gemm_small_reduce<EPI, F8, PM><<<dim3(PM * SP / 1024, pieces), dim3(256), 0, stream>>>(
      part, bias, C, ldc, M, sm, splits, alpha, oscale);
  return hipGetLastError();
}

template <Epilogue EPI, bool F8>
hipError_t launch_t(const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw, const float* bias,
                    void* C, int64_t ldc, int64_t M, int N, int K, float* part,
                    size_t part_bytes, float alpha, float oscale, hipStream_t stream) {
  const int tiles_m = (int)((M + BIG - 1) / BIG);
  const int tiles_n = N / BIG;
  const int tiles = tiles_m * tiles_n;
  const int cus = num_cus();
  // A remainder of more than a quarter of a round of tiles runs as one more,
  // partial round of the persistent kernel: as 64 x 64 pieces it takes
  // longer than one tile.  Measured (same box, alternating runs): the
  // 10-minute recording's QKV (194 remaining tiles) and attention output and
  // FFN-down products (150 tiles, one partial round), 27.90 -> 25.05 ms per
  // step; in the one-hour recording's 30-s chunks the remainders of 80
  // (QKV), 112 (O, FFN down) and 192 (FFN up) tiles, 72.09 -> 70.90 ms with
  // a half-round threshold and 69.77 -> 69.10 ms going from a third to a
  // quarter.  bf16 only, as measured.
  const bool partial_round = !F8 && (tiles % cus) * 4 > cus;
  if (tiles < cus && !partial_round) {
    // Fewer big tiles than CUs: the whole product as pieces.  Pieces of 128
    // rows move 43 instead of 32 flops per byte through the CU's load path
    // but hold one workgroup per CU (96 KB of LDS) instead of two, whose
    // start-up and epilogue then overlap nothing: they are taken when they
    // still occupy 7/8 of the CUs and each workgroup runs at least 16 K steps
    // (30-s clip, same box: FFN up 17.1 -> 15.4 us and FFN down 19.4 ->
    // 18.5 us per launch; QKV with 180 such pieces and the attention output
    // projection with 5-step splits were slower and keep 64-row pieces).
    // bf16 only: the FP8 products were not measured on them.
    if constexpr (!F8) {
      const int pieces = (int)((M + 2 * SP - 1) / (2 * SP)) * (N / SP);
      const int splits = small_splits(K, pieces, pieces, 2 * SP, cus, part_bytes);
      if (pieces * splits >= cus - cus / 8 && K / SBK / splits >= 16)
        return launch_small<EPI, F8, 2 * SP>(A, lda, W, ldw, bias, C, ldc, M, K, part,
                                             part_bytes, SmallMap{1, 0, 0, 0, N / SP}, pieces,
                                             pieces, cus, alpha, oscale, stream);
    }
    const int pieces = (int)((M + SP - 1) / SP) * (N / SP);
    return launch_small<EPI, F8, SP>(A, lda, W, ldw, bias, C, ldc, M, K, part, part_bytes,
                                     SmallMap{1, 0, 0, 0, N / SP}, pieces, pieces, cus, alpha,
                                     oscale, stream);
  }
  // Full rounds (and a partial last one) go to the persistent kernel, the
  // remainder to 64 x 64 pieces.
  const int n_big = partial_round ? tiles : (tiles / cus) * cus;
  if constexpr (EPI == Epilogue::kBiasResidualF32 && !F8) {
    if (n_big <= cus)   // one round: every CU holds at most one tile
      gemm_big_kernel<EPI, F8, true><<<dim3(cus), dim3(512), 0, stream>>>(
          A, lda, W, ldw, bias, C, ldc, M, K, tiles_m, tiles_n, n_big, alpha, oscale);
    else
      gemm_big_kernel<EPI, F8, false><<<dim3(cus), dim3(512), 0, stream>>>(
          A, lda, W, ldw, bias, C, ldc, M, K, tiles_m, tiles_n, n_big, alpha, oscale);
  } else {
    gemm_big_kernel<EPI, F8, false><<<dim3(cus), dim3(512), 0, stream>>>(
        A, lda, W, ldw, bias, C, ldc, M, K, tiles_m, tiles_n, n_big, alpha, oscale);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || tiles == n_big) return e;
  // The tail tiles as 64 x 64 pieces, sixteen per tile (measured 2.7% per
  // step faster in bf16, 3.3% in FP8, than 128 x 128 pieces with split K on
  // the 64-clip batch).
  const int pieces = 16 * (tiles - n_big);
  int live = 0;
  for (int t = n_big; t < tiles; ++t) {
    const int per_group = GROUP_M * tiles_n;
    const int first_m = (t / per_group) * GROUP_M;
    const int gsize = std::min(tiles_m - first_m, GROUP_M);
    const int64_t tm = first_m + (t - (t / per_group) * per_group) % gsize;
    live += 4 * (int)std::min<int64_t>(4, (M - tm * BIG + SP - 1) / SP);
  }
  return launch_small<EPI, F8, SP>(A, lda, W, ldw, bias, C, ldc, M, K, part, part_bytes,
                                   SmallMap{0, n_big, tiles_m, tiles_n, 0}, live, pieces, cus,
                                   alpha, oscale, stream);
}

template <bool F8>
hipError_t launch_cols(Epilogue epi, const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw,
                       const float* bias, void* C, int64_t ldc, int64_t M, int N, int K,
                       float* part, size_t part_bytes, float alpha, float oscale,
                       hipStream_t stream) {
  switch (epi) {
    case Epilogue::kBiasBf16:
      return launch_t<Epilogue::kBiasBf16, F8>(A, lda, W, ldw, bias, C, ldc, M, N, K, part,
                                               part_bytes, alpha, oscale, stream);
    case Epilogue::kBiasGeluBf16:
      return launch_t<Epilogue::kBiasGeluBf16, F8>(A, lda, W, ldw, bias, C, ldc, M, N, K, part,
                                                   part_bytes, alpha, oscale, stream);
    case Epilogue::kBiasResidualF32:
      return launch_t<Epilogue::kBiasResidualF32, F8>(A, lda, W, ldw, bias, C, ldc, M, N, K, part,
                                                      part_bytes, alpha, oscale, stream);
    case Epilogue::kBiasF32:
      return launch_t<Epilogue::kBiasF32, F8>(A, lda, W, ldw, bias, C, ldc, M, N, K, part,
                                              part_bytes, alpha, oscale, stream);
    case Epilogue::kBiasGeluFp8:
      if constexpr (F8)
        return launch_t<Epilogue::kBiasGeluFp8, true>(A, lda, W, ldw, bias, C, ldc, M, N, K, part,
                                                      part_bytes, alpha, oscale, stream);
      break;
  }
  return hipErrorInvalidValue;
}

// Whole 256-column tiles first; a last strip of 128 columns (N % 256 == 128)
// is a product of its own (on the 64 x 64 pieces).  c_elem: bytes per C element.
template <bool F8>
hipError_t launch_split_n(Epilogue epi, const bf16_t* A, int64_t lda, const bf16_t* W,
                          int64_t ldw, const float* bias, void* C, int64_t ldc, int64_t M, int N,
                          int K, float* part, size_t part_bytes, float alpha, float oscale,
                          size_t c_elem, hipStream_t stream) {
  const int n_main = N / BIG * BIG;
  hipError_t e = hipSuccess;
  if (n_main > 0)
    e = launch_cols<F8>(epi, A, lda, W, ldw, bias, C, ldc, M, n_main, K, part, part_bytes, alpha,
                        oscale, stream);
  if (e != hipSuccess || n_main == N) return e;
  return launch_cols<F8>(epi, A, lda, W + (int64_t)n_main * ldw, ldw, bias + n_main,
                         (char*)C + (size_t)n_main * c_elem, ldc, M, N - n_main, K, part,
                         part_bytes, alpha, oscale, stream);
}

}  // namespace

int num_cus() {
  static int n_cus = 0;
  if (n_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      n_cus = n;
    else
      n_cus = 256;
  }
  return n_cus;
}

hipError_t launch_gemm(Epilogue epi, const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw,
                       const float* bias, void* C, int64_t ldc, int64_t M, int N, int K,
                       float* part, size_t part_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  // N in 128-column strips, K in whole 64-wide steps of both kernels (the
  // documented contract asks K % 256 == 0)
  if (N <= 0 || N % 128 != 0 || K % 256 != 0 || epi == Epilogue::kBiasGeluFp8)
    return hipErrorInvalidValue;
  const size_t c_elem = (epi == Epilogue::kBiasBf16 || epi == Epilogue::kBiasGeluBf16) ? 2 : 4;
  return launch_split_n<false>(epi, A, lda, W, ldw, bias, C, ldc, M, N, K, part, part_bytes, 1.0f,
                               1.0f, c_elem, stream);
}

hipError_t launch_gemm_fp8(Epilogue epi, const uint8_t* A, int64_t lda, const uint8_t* W,
                           int64_t ldw, float alpha, float out_scale, const float* bias, void* C,
                           int64_t ldc, int64_t M, int N, int K, float* part, size_t part_bytes,
                           hipStream_t stream) {
  if (M == 0) return hipSuccess;
  // Codes are moved as pairs (bf16-sized units): K / 2 must be a whole number
  // of 64-wide steps (K % 256 codes, as documented) and the strides even.
  if (N <= 0 || N % 128 != 0 || K % 256 != 0 || (lda & 1) || (ldw & 1) ||
      epi == Epilogue::kBiasGeluBf16)
    return hipErrorInvalidValue;
  const size_t c_elem = epi == Epilogue::kBiasGeluFp8 ? 1 : epi == Epilogue::kBiasBf16 ? 2 : 4;
  return launch_split_n<true>(epi, reinterpret_cast<const bf16_t*>(A), lda / 2,
                              reinterpret_cast<const bf16_t*>(W), ldw / 2, bias, C, ldc, M, N,
                              K / 2, part, part_bytes, alpha, out_scale, c_elem, stream);
}

}  // namespace enc
