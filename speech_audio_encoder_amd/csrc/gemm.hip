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
//  * gemm_splitk_kernel + splitk_reduce_kernel -- the tiles left after the
//    last full round, cut into 128 x 128 pieces and split along K so that the
//    final partial round spreads over every CU (a 256 x 256 tile per CU would
//    leave most CUs idle for a whole tile time).
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
  const int S = my_tiles * KT;

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

// ------------------------------------------------------------- tail (split K)
// The tiles left after the last full round: each 256 x 256 tile is cut into
// four 128 x 128 pieces and K into `splits` equal ranges, so that the tail
// occupies every CU for a short time instead of a few CUs for a whole tile.
// Each workgroup writes its fp32 partial sums; splitk_reduce_kernel adds the
// partials of a piece in a fixed order (deterministic) and applies the
// epilogue.  128 x 128 per workgroup, four wavefronts of 64 x 64, K in steps
// of 64 through registers (two steps in flight) and one LDS buffer.
constexpr int SBK = 64;
constexpr int PIECE = 128;

__global__ __launch_bounds__(256) void gemm_splitk_kernel(
    const bf16_t* __restrict__ A, int64_t lda, const bf16_t* __restrict__ W, int64_t ldw,
    float* __restrict__ part, int64_t M, int K, int tiles_m, int tiles_n, int t_begin,
    int splits) {
  constexpr int CH = PIECE * SBK / 8;        // 16-byte chunks per operand tile
  __shared__ uint4 sA[CH];
  __shared__ uint4 sW[CH];

  const int split = blockIdx.x % splits;
  const int pid = blockIdx.x / splits;       // piece index
  const int piece = pid & 3;
  int tm, tn;
  tile_coords(t_begin + (pid >> 2), tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BIG + (piece & 1) * PIECE;
  const int64_t n0 = (int64_t)tn * BIG + (piece >> 1) * PIECE;
  const int kc = K / splits;
  const int kb = split * kc;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;

  const bf16_t* ap[4];
  const bf16_t* wp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * 256;
    const int row = c >> 3, col = (c & 7) * 8;
    ap[i] = A + min<int64_t>(m0 + row, M - 1) * lda + kb + col;
    wp[i] = W + (n0 + row) * ldw + kb + col;
  }
  uint4 ra[2][4], rw[2][4];
  auto load_regs = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[buf][i] = *reinterpret_cast<const uint4*>(ap[i] + k0);
      rw[buf][i] = *reinterpret_cast<const uint4*>(wp[i] + k0);
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int row = c >> 3, ch = c & 7;
      sA[row * 8 + (ch ^ (row & 7))] = ra[buf][i];
      sW[row * 8 + (ch ^ (row & 7))] = rw[buf][i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int steps = kc / SBK;
  load_regs(0, 0);
  if (steps > 1) load_regs(SBK, 1);
  for (int st = 0; st < steps; ++st) {
    __syncthreads();
    if (st & 1) store_tiles(1); else store_tiles(0);
    __syncthreads();
    if (st + 2 < steps) {
      if (st & 1) load_regs((st + 2) * SBK, 1); else load_regs((st + 2) * SBK, 0);
    }
#pragma unroll
    for (int s = 0; s < SBK / 16; ++s) {
      const int chunk = 2 * s + lhi;
      bf16x8 fw[2], fa[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wn * 64 + i * 32 + l32;
        const uint4 u = sW[row * 8 + (chunk ^ (row & 7))];
        fw[i] = *reinterpret_cast<const bf16x8*>(&u);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = wm * 64 + j * 32 + l32;
        const uint4 u = sA[row * 8 + (chunk ^ (row & 7))];
        fa[j] = *reinterpret_cast<const bf16x8*>(&u);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[i], fa[j], acc[i][j], 0, 0, 0);
    }
  }

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
}

// Sum the split partials of each piece (split order 0, 1, ...) and apply the
// epilogue.  One thread per 4 consecutive columns.
template <Epilogue EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, void* __restrict__ Cv,
    int64_t ldc, int64_t M, int tiles_m, int tiles_n, int t_begin, int splits) {
  const int pid = blockIdx.y;
  const int piece = pid & 3;
  int tm, tn;
  tile_coords(t_begin + (pid >> 2), tiles_m, tiles_n, tm, tn);
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;   // element in the piece
  const int r = e / PIECE, c = e % PIECE;
  const int64_t m = (int64_t)tm * BIG + (piece & 1) * PIECE + r;
  const int n = tn * BIG + (piece >> 1) * PIECE + c;
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

template <Epilogue EPI>
hipError_t launch_t(const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw, const float* bias,
                    void* C, int64_t ldc, int64_t M, int N, int K, float* part,
                    size_t part_bytes, hipStream_t stream) {
  const int tiles_m = (int)((M + BIG - 1) / BIG);
  const int tiles_n = N / BIG;
  const int tiles = tiles_m * tiles_n;
  const int cus = num_cus();
  // Full rounds go to the persistent kernel, the remainder to the split-K tail.
  const int n_big = (tiles / cus) * cus;
  if (n_big > 0) {
    if ((K / BKS) % 10 == 0)
      gemm_big_kernel<EPI, 5><<<dim3(cus), dim3(256), 0, stream>>>(A, lda, W, ldw, bias, C, ldc, M,
                                                                   K, tiles_m, tiles_n, n_big);
    else
      gemm_big_kernel<EPI, 4><<<dim3(cus), dim3(256), 0, stream>>>(A, lda, W, ldw, bias, C, ldc, M,
                                                                   K, tiles_m, tiles_n, n_big);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (tiles > n_big) {
    // Split K so that pieces x splits fills about two workgroups per CU, each
    // with at least two 64-wide steps, within the partial buffer.
    const int pieces = 4 * (tiles - n_big);
    const int kblocks = K / SBK;
    int splits = 1;
    for (int sp = 2; sp <= kblocks / 2; ++sp) {
      if (kblocks % sp) continue;
      if ((int64_t)pieces * sp > 2 * cus) break;
      if ((size_t)pieces * sp * PIECE * PIECE * sizeof(float) > part_bytes) break;
      splits = sp;
    }
    if ((size_t)pieces * splits * PIECE * PIECE * sizeof(float) > part_bytes)
      return hipErrorInvalidValue;
    gemm_splitk_kernel<<<dim3(pieces * splits), dim3(256), 0, stream>>>(
        A, lda, W, ldw, part, M, K, tiles_m, tiles_n, n_big, splits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    splitk_reduce_kernel<EPI><<<dim3(PIECE * PIECE / 1024, pieces), dim3(256), 0, stream>>>(
        part, bias, C, ldc, M, tiles_m, tiles_n, n_big, splits);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm(Epilogue epi, const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw,
                       const float* bias, void* C, int64_t ldc, int64_t M, int N, int K,
                       float* part, size_t part_bytes, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  if (N % BIG != 0 || K % (BKS * 8) != 0 || K % SBK != 0) return hipErrorInvalidValue;
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
