// bf16 MFMA GEMM for gfx950 with fused epilogues:
//   C[M, N] (op)= A[M, K] * W[N, K]^T + bias
// A holds activations (rows = packed positions), W a weight matrix in the
// [out, in] layout, both K-contiguous, fp32 accumulation.
//
// Used for the input projection (width 1024 -> 1280), the fused QKV
// projection, the attention output projection and the two FFN matrices of
// "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
// "How audio and speakers reach the language model" (width 1,280, feed-forward
// expansion four; exact-erf GELU is this build's reading of the activation).
//
// Two kernels share the output tiling (256 x 256 tiles, numbered in groups of
// four tile rows so that neighbouring tiles share A rows and W columns):
//
//  * gemm_big_kernel -- persistent, one workgroup per CU, four wavefronts of
//    128 x 128 outputs each (16 MFMA 32x32x16 accumulators, held in AGPRs).
//    It covers every full round of tiles.  Operands go straight from global
//    memory into LDS with global_load_lds_dwordx4 (no register staging; the
//    XOR swizzle that keeps the MFMA operand reads conflict-free is applied on
//    the global side by choosing which 16-byte chunk each lane fetches).  A
//    four-stage ring of 32-wide K steps (4 x 32 KB) keeps three steps of loads
//    in flight; one barrier per step.  The stream of steps runs on across the
//    workgroup's tiles, so the next tile's loads overlap this tile's epilogue.
//  * gemm_piece_kernel (+ splitk_reduce_kernel) -- the tiles left after the
//    last full round, or the whole product when it has fewer 256 x 256 tiles
//    than CUs, as 128 x 128 pieces split along K when needed so that every CU
//    is busy (a 256 x 256 tile per CU would leave most CUs idle).
//
// Each lane ends up owning one output row and runs of four consecutive
// columns: the epilogue adds bias / residual / GELU in registers and stores
// 8- or 16-byte vectors.

#include <cstdlib>

#include "common.h"
#include "kernels.h"

namespace enc {

namespace {

constexpr int BIG = 256;    // big tile edge
constexpr int BKS = 32;     // big kernel K step
constexpr int GROUP_M = 4;  // tile rows per ordering group

// Exact-erf GELU, x Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), with erf taken from
// Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erf(z) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2),
// t = 1 / (1 + p z), z >= 0, absolute error below 1.5e-7 -- far below the
// bf16 rounding of the output -- at one reciprocal, one exponential and five
// fused multiply-adds instead of a general-purpose erf.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, z, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  const float e = 1.0f - poly * __expf(-z * z);      // erf(|x| / sqrt 2)
  const float phi2 = x >= 0.0f ? 1.0f + e : 1.0f - e;  // 2 Phi(x)
  return 0.5f * x * phi2;
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
template <Epilogue EPI>
__device__ __forceinline__ void store4(void* __restrict__ Cv, int64_t ldc, int64_t m, int n,
                                       float4 bv, float a0, float a1, float a2, float a3) {
  float o0 = a0 + bv.x, o1 = a1 + bv.y, o2 = a2 + bv.z, o3 = a3 + bv.w;
  if constexpr (EPI == Epilogue::kBiasGeluBf16) {
    o0 = gelu_erf(o0); o1 = gelu_erf(o1); o2 = gelu_erf(o2); o3 = gelu_erf(o3);
  }
  if constexpr (EPI == Epilogue::kBiasBf16 || EPI == Epilogue::kBiasGeluBf16) {
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

// ----------------------------------------------------------- big (persistent)
template <Epilogue EPI, int NS>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ bias, void* __restrict__ Cv, int64_t ldc, int64_t M, int K,
    int tiles_m, int tiles_n, int n_big) {
  // Stage layout (uint4 units): A rows 0..255 x 4 chunks, then W rows x 4.
  constexpr int STG = 2 * BIG * BKS / 8;
  // NS stages of 32 KB.  Distinct arrays, referenced statically, so the
  // compiler can tell a DMA into one stage from reads of another and does not
  // wait on it (unused ones are not allocated).
  static_assert(NS == 4 || NS == 5, "ring depth");
  __shared__ uint4 st0[STG];
  __shared__ uint4 st1[STG];
  __shared__ uint4 st2[STG];
  __shared__ uint4 st3[STG];
  __shared__ uint4 st4[STG];
  auto stage = [&](int i) -> uint4* {
    switch (i) {
      case 0: return st0;
      case 1: return st1;
      case 2: return st2;
      case 3: return st3;
      default: return st4;
    }
  };

  const int G = gridDim.x;
  const int wg = blockIdx.x;
  // Hardware block wg runs on XCD wg % 8: give each XCD a contiguous slot range.
  const int slot = (G % 8 == 0) ? (wg % 8) * (G / 8) + wg / 8 : wg;
  const int my_tiles = slot < n_big ? (n_big - 1 - slot) / G + 1 : 0;
  const int KT = K / BKS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // DMA lane mapping: wavefront load i of wave w covers tile rows
  // (w*4 + i)*16 + lane/4 (16 rows of 64 B); lane%4 is the physical chunk,
  // holding logical chunk (lane%4) ^ ((row/2) % 4).
  const int drow = wave * 64 + (lane >> 2);
  const int dcol = ((lane & 3) ^ ((lane >> 3) & 3)) * 8;
  // Issue state: tile ir of this workgroup, k step ikt, and the per-lane
  // source rows of that tile (rows past M re-read row M-1; dropped later).
  // Past the workgroup's last tile the loads simply repeat that tile's K
  // range (harmless, and it keeps the step body free of branches).
  int ir = 0, ikt = 0;
  const bf16_t* ia[4];
  const bf16_t* iw[4];
  auto set_issue_tile = [&]() {
    int tm, tn;
    tile_coords(min(ir, my_tiles - 1) * G + slot, tiles_m, tiles_n, tm, tn);
    const int64_t am = (int64_t)tm * BIG;
    const int64_t wn0 = (int64_t)tn * BIG;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ia[i] = A + min<int64_t>(am + drow + 16 * i, M - 1) * lda + dcol;
      iw[i] = W + (wn0 + drow + 16 * i) * ldw + dcol;
    }
  };
  auto issue = [&](uint4* stage) {
    const int k0 = ikt * BKS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dma16(ia[i] + k0, (lds_void*)(stage + (wave * 4 + i) * 64));
      dma16(iw[i] + k0, (lds_void*)(stage + BIG * 4 + (wave * 4 + i) * 64));
    }
  };
  auto advance = [&]() {
    if (++ikt == KT) {
      ikt = 0;
      ++ir;
      if (ir < my_tiles) set_issue_tile();
    }
  };

  // Operand reads: row r of a stage, logical chunk c -> uint4 r*4 + (c ^ ((r/2)%4)).
  const int rsw = (l32 >> 1) & 3;
  const int wofs = BIG * 4 + (wn * 128 + l32) * 4;
  const int aofs = (wm * 128 + l32) * 4;

  f32x16 acc[4][4];
  // Operand fragments of a whole 32-wide step (two 16-wide slices: 4 of W and
  // 4 of A each), double-buffered across steps.
  bf16x8 fb0[16], fb1[16];
  auto load = [&](const uint4* sp, bf16x8 (&f)[16]) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      const int pc = (2 * sl + lhi) ^ rsw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 u = sp[wofs + i * 128 + pc];
        f[sl * 8 + i] = *reinterpret_cast<const bf16x8*>(&u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 u = sp[aofs + j * 128 + pc];
        f[sl * 8 + 4 + j] = *reinterpret_cast<const bf16x8*>(&u);
      }
    }
  };
  auto mma = [&](const bf16x8 (&f)[16]) {
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[sl * 8 + i], f[sl * 8 + 4 + j],
                                                              acc[i][j], 0, 0, 0);
  };
  // Within one basic block, spread the 16 LDS reads of step g between the 32
  // MFMAs of step g - 1 (a wave that issues an MFMA can issue an LDS read
  // while the matrix core works; a burst of reads would leave it idle).  The
  // 8 DMAs of step g + NS - 1 go out as one burst before the MFMAs: spread
  // between them they measured slower.
  auto interleave = [&]() {
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // MFMA
    }
  };

  set_issue_tile();
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) {
    issue(stage(i));
    advance();
  }
  int since_epi = 0;   // steps since the last epilogue (its stores count in vmcnt)

  // s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
  // 6:4, lgkmcnt 11:8); fields not named are left at their maximum.
  // WAIT_STEP allows the loads of the NS - 2 younger steps (8 DMAs each).
  constexpr int WAIT_LGKM0 = 0xC07F;                       // lgkmcnt(0)
  constexpr int VM = 8 * (NS - 2);
  constexpr int WAIT_STEP = (VM & 15) | ((VM >> 4) << 14) | 0x0070;  // vmcnt(VM) lgkmcnt(0)
  constexpr int WAIT_EPI = 0xC07F & ~0x0F00;               // vmcnt(63) lgkmcnt(0)

  // One K step (tile-local index u) on stage u % NS: its fragments go to
  // fb[u % 2] while the MFMAs of the previous step run from the other buffer
  // (none on a tile's first step), and the loads of the step NS - 1 ahead go
  // to the stage just freed.  Before the barrier each wave waits for its own
  // loads of this step (the younger steps stay in flight; just after an
  // epilogue its stores count too, hence the looser bound) and for its LDS
  // reads of the previous step, whose stage the new loads overwrite.  The
  // barrier is the bare s_barrier: a fenced one would also wait for the
  // younger loads.
  auto step = [&](int u, bool first) {
    if (since_epi > 0 && since_epi < NS)
      __builtin_amdgcn_s_waitcnt(WAIT_EPI);
    else
      __builtin_amdgcn_s_waitcnt(WAIT_STEP);
    __builtin_amdgcn_s_barrier();
    issue(stage((u + NS - 1) % NS));
    if (u & 1) load(stage(u % NS), fb1); else load(stage(u % NS), fb0);
    if (!first) {
      if (u & 1) mma(fb0); else mma(fb1);
      interleave();
    }
    advance();
    if (since_epi > 0) ++since_epi;
  };

  for (int r = 0; r < my_tiles; ++r) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    // K / 32 is a multiple of 2 * NS: the stage and fragment buffer of every
    // step are compile-time constants in the unrolled body.
#pragma unroll
    for (int u = 0; u < 2 * NS; ++u) step(u, u == 0);
    for (int kt = 2 * NS; kt < KT; kt += 2 * NS) {
#pragma unroll
      for (int u = 0; u < 2 * NS; ++u) step(u, false);
    }
    __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
    mma(fb1);

    int tm, tn;
    tile_coords(r * G + slot, tiles_m, tiles_n, tm, tn);
    const int64_t mb = (int64_t)tm * BIG + wm * 128 + l32;
    const int nw = tn * BIG + wn * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 bv[4];
      load_bias32(bias, nw + i * 32, lhi, bv);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t m = mb + j * 32;
        if (m < M) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            store4<EPI>(Cv, ldc, m, nw + i * 32 + 8 * q + 4 * lhi, bv[q], acc[i][j][4 * q],
                        acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
    }
    since_epi = 1;
  }
  // Loads past the last step may still be landing in LDS: drain them before
  // the workgroup's LDS is released.
  __builtin_amdgcn_s_waitcnt(0);
}

// ------------------------------------------------------- 128 x 128 pieces
// Work the persistent kernel does not cover -- the tiles left after its last
// full round, or the whole product when there are fewer 256 x 256 tiles than
// CUs -- is cut into 128 x 128 pieces, and K into `splits` ranges when that
// is needed to occupy every CU.  A workgroup (four wavefronts of 64 x 64)
// takes one (piece, split): the same direct-to-LDS ring as the big kernel,
// 4 stages of 32-wide K steps (16 KB each), so two workgroups fit on a CU and
// cover each other's waits.  With one split the epilogue is applied directly;
// otherwise fp32 partial sums go to `part` and splitk_reduce_kernel adds them
// in a fixed order (deterministic) and applies the epilogue.
constexpr int PIECE = 128;
constexpr int PNS = 4;

struct PieceMap {
  int mode;       // 0: pieces of leftover big tiles t_begin.., 1: a plain grid
  int t_begin;    // mode 0
  int tiles_m, tiles_n;
  int pieces_n;   // mode 1: pieces per row of pieces (N / 128)
};

__device__ __forceinline__ void piece_coords(int pid, const PieceMap& pm, int64_t& m0, int64_t& n0) {
  if (pm.mode == 0) {
    int tm, tn;
    tile_coords(pm.t_begin + (pid >> 2), pm.tiles_m, pm.tiles_n, tm, tn);
    m0 = (int64_t)tm * BIG + (pid & 1) * PIECE;
    n0 = (int64_t)tn * BIG + ((pid >> 1) & 1) * PIECE;
  } else {
    // groups of 8 piece rows, column-major inside a group
    const int per_group = 8 * pm.pieces_n;
    const int group = pid / per_group;
    const int pieces_m = (pm.tiles_m * BIG) / PIECE;   // rounded up to whole big tiles
    const int first = group * 8;
    const int gsize = min(pieces_m - first, 8);
    const int r = pid - group * per_group;
    m0 = (int64_t)(first + r % gsize) * PIECE;
    n0 = (int64_t)(r / gsize) * PIECE;
  }
}

template <Epilogue EPI, bool PARTIAL>
__global__ __launch_bounds__(256, 2) void gemm_piece_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ bias, void* __restrict__ Cv, int64_t ldc, float* __restrict__ part,
    int64_t M, int K, PieceMap pm, int splits) {
  constexpr int STG = 2 * PIECE * BKS / 8;   // uint4 per stage (16 KB)
  __shared__ uint4 st0[STG];
  __shared__ uint4 st1[STG];
  __shared__ uint4 st2[STG];
  __shared__ uint4 st3[STG];
  auto stage = [&](int i) -> uint4* {
    switch (i & 3) {
      case 0: return st0;
      case 1: return st1;
      case 2: return st2;
      default: return st3;
    }
  };

  const int split = blockIdx.x % splits;
  const int pid = blockIdx.x / splits;
  int64_t m0, n0;
  piece_coords(pid, pm, m0, n0);
  if (m0 >= M) return;   // whole piece past the last row (plain grid rounding)
  const int kc = K / splits;
  const int kb = split * kc;
  const int KT = kc / BKS;   // multiple of PNS

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  // DMA: wave w loads 2 x 16 rows of A and of W per step (rows (w*2+i)*16 + lane/4).
  const int drow = wave * 32 + (lane >> 2);
  const int dcol = ((lane & 3) ^ ((lane >> 3) & 3)) * 8;
  const bf16_t* ia[2];
  const bf16_t* iw[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ia[i] = A + min<int64_t>(m0 + drow + 16 * i, M - 1) * lda + kb + dcol;
    iw[i] = W + (n0 + drow + 16 * i) * ldw + kb + dcol;
  }
  int ikt = 0;
  auto issue = [&](uint4* sp) {
    const int k0 = min(ikt, KT - 1) * BKS;   // past the end: re-read the last step
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      dma16(ia[i] + k0, (lds_void*)(sp + (wave * 2 + i) * 64));
      dma16(iw[i] + k0, (lds_void*)(sp + PIECE * 4 + (wave * 2 + i) * 64));
    }
    ++ikt;
  };

  const int rsw = (l32 >> 1) & 3;
  const int wofs = PIECE * 4 + (wn * 64 + l32) * 4;
  const int aofs = (wm * 64 + l32) * 4;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  constexpr int VM = 4 * (PNS - 2);
  constexpr int WAIT_STEP = (VM & 15) | ((VM >> 4) << 14) | 0x0070;   // vmcnt(8) lgkmcnt(0)
#pragma unroll
  for (int i = 0; i < PNS - 1; ++i) issue(stage(i));
  for (int kt = 0; kt < KT; kt += PNS) {
#pragma unroll
    for (int u = 0; u < PNS; ++u) {
      __builtin_amdgcn_s_waitcnt(WAIT_STEP);
      __builtin_amdgcn_s_barrier();
      issue(stage(u + PNS - 1));
      const uint4* sp = stage(u);
      bf16x8 fw[2][2], fa[2][2];
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        const int pc = (2 * sl + lhi) ^ rsw;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 uw = sp[wofs + i * 128 + pc];
          fw[sl][i] = *reinterpret_cast<const bf16x8*>(&uw);
          const uint4 ua = sp[aofs + i * 128 + pc];
          fa[sl][i] = *reinterpret_cast<const bf16x8*>(&ua);
        }
      }
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[sl][i], fa[sl][j], acc[i][j], 0,
                                                                0, 0);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // loads past the last step land before LDS is released

  if constexpr (PARTIAL) {
    // Partial layout: [pid][split][128 rows][128 cols] fp32.
    float* dst = part + ((int64_t)pid * splits + split) * (PIECE * PIECE);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wm * 64 + j * 32 + l32;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * 64 + i * 32 + 8 * q + 4 * lhi;
          *reinterpret_cast<float4*>(dst + r * PIECE + c) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                          acc[i][j][4 * q + 3]);
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int nw = (int)(n0 + wn * 64 + i * 32);
      float4 bv[4];
      load_bias32(bias, nw, lhi, bv);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t m = m0 + wm * 64 + j * 32 + l32;
        if (m >= M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          store4<EPI>(Cv, ldc, m, nw + 8 * q + 4 * lhi, bv[q], acc[i][j][4 * q],
                      acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
    }
  }
}

// Sum the split partials of each piece (split order 0, 1, ...) and apply the
// epilogue.  One thread per 4 consecutive columns.
template <Epilogue EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, void* __restrict__ Cv,
    int64_t ldc, int64_t M, PieceMap pm, int splits) {
  const int pid = blockIdx.y;
  int64_t m0, n0;
  piece_coords(pid, pm, m0, n0);
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;   // element in the piece
  const int r = e / PIECE, c = e % PIECE;
  const int64_t m = m0 + r;
  const int n = (int)n0 + c;
  if (m >= M) return;
  const float* src = part + (int64_t)pid * splits * (PIECE * PIECE) + e;
  float4 s = *reinterpret_cast<const float4*>(src);
  for (int k = 1; k < splits; ++k) {
    const float4 t = *reinterpret_cast<const float4*>(src + (int64_t)k * (PIECE * PIECE));
    s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
  }
  store4<EPI>(Cv, ldc, m, n, *reinterpret_cast<const float4*>(bias + n), s.x, s.y, s.z, s.w);
}

int g_num_cus = 0;

int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

// Split K (into a divisor of K / 128 ranges) as far as the pieces that hold
// rows stay within two workgroups per CU, and the partial sums of every piece
// id within the partial buffer.
int choose_splits(int live_pieces, int grid_pieces, int K, int cus, size_t part_bytes) {
  const int units = K / (BKS * PNS);
  int splits = 1;
  for (int sp = 2; sp <= units; ++sp) {
    if (units % sp) continue;
    if ((int64_t)live_pieces * sp > 2 * cus) break;
    if ((size_t)grid_pieces * sp * PIECE * PIECE * sizeof(float) > part_bytes) break;
    splits = sp;
  }
  return splits;
}

template <Epilogue EPI>
hipError_t launch_pieces(const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw,
                         const float* bias, void* C, int64_t ldc, int64_t M, int K, float* part,
                         size_t part_bytes, const PieceMap& pm, int live_pieces, int pieces,
                         int cus, hipStream_t stream) {
  const int splits = choose_splits(live_pieces, pieces, K, cus, part_bytes);
  if (splits == 1) {
    gemm_piece_kernel<EPI, false><<<dim3(pieces), dim3(256), 0, stream>>>(
        A, lda, W, ldw, bias, C, ldc, part, M, K, pm, 1);
    return hipGetLastError();
  }
  gemm_piece_kernel<EPI, true><<<dim3(pieces * splits), dim3(256), 0, stream>>>(
      A, lda, W, ldw, bias, C, ldc, part, M, K, pm, splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  splitk_reduce_kernel<EPI><<<dim3(PIECE * PIECE / 1024, pieces), dim3(256), 0, stream>>>(
      part, bias, C, ldc, M, pm, splits);
  return hipGetLastError();
}

template <Epilogue EPI>
hipError_t launch_t(const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw, const float* bias,
                    void* C, int64_t ldc, int64_t M, int N, int K, float* part,
                    size_t part_bytes, hipStream_t stream) {
  const int tiles_m = (int)((M + BIG - 1) / BIG);
  const int tiles_n = N / BIG;
  const int tiles = tiles_m * tiles_n;
  const int cus = num_cus();
  if (tiles < cus) {
    // Fewer big tiles than CUs: the whole product as 128 x 128 pieces.
    PieceMap pm{1, 0, tiles_m, tiles_n, N / PIECE};
    const int live = (int)((M + PIECE - 1) / PIECE) * (N / PIECE);
    // piece ids cover whole big-tile rows; ids past M return at once
    const int grid_pieces = ((tiles_m * BIG) / PIECE) * (N / PIECE);
    return launch_pieces<EPI>(A, lda, W, ldw, bias, C, ldc, M, K, part, part_bytes, pm, live,
                              grid_pieces, cus, stream);
  }
  // Full rounds go to the persistent kernel, the remainder to 128 x 128 pieces.
  const int n_big = (tiles / cus) * cus;
  if ((K / BKS) % 10 == 0)
    gemm_big_kernel<EPI, 5><<<dim3(cus), dim3(256), 0, stream>>>(A, lda, W, ldw, bias, C, ldc, M,
                                                                 K, tiles_m, tiles_n, n_big);
  else
    gemm_big_kernel<EPI, 4><<<dim3(cus), dim3(256), 0, stream>>>(A, lda, W, ldw, bias, C, ldc, M,
                                                                 K, tiles_m, tiles_n, n_big);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || tiles == n_big) return e;
  PieceMap pm{0, n_big, tiles_m, tiles_n, N / PIECE};
  return launch_pieces<EPI>(A, lda, W, ldw, bias, C, ldc, M, K, part, part_bytes, pm,
                            4 * (tiles - n_big), 4 * (tiles - n_big), cus, stream);
}

}  // namespace

hipError_t launch_gemm(Epilogue epi, const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw,
                       const float* bias, void* C, int64_t ldc, int64_t M, int N, int K,
                       float* part, size_t part_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (N % BIG != 0 || K % (BKS * 8) != 0) return hipErrorInvalidValue;
  switch (epi) {
    case Epilogue::kBiasBf16:
      return launch_t<Epilogue::kBiasBf16>(A, lda, W, ldw, bias, C, ldc, M, N, K, part, part_bytes,
                                           stream);
    case Epilogue::kBiasGeluBf16:
      return launch_t<Epilogue::kBiasGeluBf16>(A, lda, W, ldw, bias, C, ldc, M, N, K, part,
                                               part_bytes, stream);
    case Epilogue::kBiasResidualF32:
      return launch_t<Epilogue::kBiasResidualF32>(A, lda, W, ldw, bias, C, ldc, M, N, K, part,
                                                  part_bytes, stream);
    case Epilogue::kBiasF32:
      return launch_t<Epilogue::kBiasF32>(A, lda, W, ldw, bias, C, ldc, M, N, K, part, part_bytes,
                                          stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace enc
