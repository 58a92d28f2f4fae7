// Internal interface between the host runtime and the gfx950 kernels.
// Every launcher is asynchronous on the given stream and returns the launch
// status; shapes are validated by the caller before anything is enqueued.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace enc {

struct Cpx {
  double re, im;
};

// Mel bands are summed by 16 lanes per frame: lane j takes bands j + 16 i
// (i = 0..7), and band group i reads MEL_GROUP_TRIP[i] consecutive bins (the
// widest band of the group; narrower bands carry zero weights).
constexpr int MEL_GROUPS = 8;
constexpr int MEL_GROUP_TRIP[MEL_GROUPS] = {2, 2, 2, 3, 4, 6, 9, 12};
constexpr int MEL_TRIP_TOTAL = 40;

// Constant tables of the frontend, built on the host in float64.
struct FrontendTables {
  double hann[WIN + 16];        // periodic Hann window, zero past WIN
  Cpx tw256[256];               // exp(-2 pi i m / 256)
  Cpx tw512[NBIN + 1];          // exp(-2 pi i k / 512), k = 0..256 (+1 pad)
  int32_t mel_rstart[NMEL];     // first bin read for band m (<= NBIN - trip)
  // weight / 4 of bin mel_rstart[m] + t for band m = j + 16 i, at row
  // (sum of the trips of groups before i) + t, column j; float32
  float mel_w4[MEL_TRIP_TOTAL][16];
};

// ---------------------------------------------------------------- frontend
// Log-mel of every (clip, frame) pair into out[batch, f_max, 128] (float32),
// zero for frames t >= n_frames[b].
hipError_t launch_logmel_padded(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                int batch, int64_t f_max, const FrontendTables* tab, float* out,
                                hipStream_t stream);

// Log-mel in the stacked layout the input projection reads: clip b owns
// packed frames [frame_base[b], frame_base[b] + 8 P_b); frames past F_b are 0.
// out is bf16 [total_frames, 128] == [sum P_b, 1024].
hipError_t launch_logmel_stacked(const float* audio, int64_t audio_stride, const int32_t* n_frames,
                                 const int32_t* frame_base, int batch, int64_t total_frames,
                                 const FrontendTables* tab, bf16_t* out, hipStream_t stream);

// -------------------------------------------------------------------- GEMM
// C[M, N] (op)= A[M, K] * W[N, K]^T + bias[N]; A, W bf16 row-major
// (K contiguous), fp32 accumulation.  N % 128 == 0, K % 256 == 0.
// `part` is scratch for split-K partial sums (GEMM_PARTIAL_BYTES suffices);
// calls on one stream may share it.
enum class Epilogue {
  kBiasBf16,          // C (bf16)  = acc + bias
  kBiasGeluBf16,      // C (bf16)  = gelu(acc + bias)
  kBiasResidualF32,   // C (fp32) += acc + bias
  kBiasF32,           // C (fp32)  = acc + bias
  kBiasGeluFp8,       // C (E4M3)  = q(gelu(acc + bias) * out_scale)   (FP8 path only)
};

constexpr size_t GEMM_PARTIAL_BYTES = (size_t)2 * 512 * 128 * 128 * sizeof(float);

// Compute units of the current device (queried once).
int num_cus();

hipError_t launch_gemm(Epilogue epi, const bf16_t* A, int64_t lda, const bf16_t* W, int64_t ldw,
                       const float* bias, void* C, int64_t ldc, int64_t M, int N, int K,
                       float* part, size_t part_bytes, hipStream_t stream);

// ------------------------------------------------------------------- norms
// y[r, :] = LN(x[r, :]) * g + b over d = 1280, fp32 statistics, bf16 output.
hipError_t launch_layernorm(const float* x, const float* g, const float* b, bf16_t* y,
                            int64_t rows, hipStream_t stream);
// The same with E4M3 output: y8[r, :] = q(LN(x[r, :]) * g + b) * out_scale).
hipError_t launch_layernorm_fp8(const float* x, const float* g, const float* b, float out_scale,
                                uint8_t* y8, int64_t rows, hipStream_t stream);

// amax[slot] = max(amax[slot], max |x|) over n bf16 values (n % 8 == 0);
// amax holds non-negative floats, so their bit patterns order as integers.
hipError_t launch_amax_bf16(const bf16_t* x, int64_t n, float* amax, hipStream_t stream);
// Per-tensor E4M3 quantization of a bf16 matrix: s = amax / 448 (1 if amax is
// 0) is read from *amax and written to *scale; q = e4m3(sat(w * (1 / s))).
hipError_t launch_quantize_fp8(const bf16_t* w, int64_t n, const float* amax, float* scale,
                               uint8_t* q, hipStream_t stream);
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t stream);

// out[r, c] = z[r, c] - log(sum_c' exp(z[r, c'])) over c, c' < n; z rows of
// stride ldz (a multiple of 4), out rows of stride n (fp32); n <= 24,576.
hipError_t launch_log_softmax(const float* z, int64_t ldz, int64_t rows, int n, float* out,
                              hipStream_t stream);

// In place on qkv bf16, per attention tile and head:
// q <- RoPE(LN_q(q)), k <- RoPE(LN_k(k)) * log2(e) / sqrt(head_dim).
// tile_info holds four int32 per tile: the sequence's first row, its length,
// the tile's first position (the tile covers positions p0 .. p0 + 127 of the
// sequence), 0.  qkv rows hold q, k, v blocks of n_heads x head_dim (row
// stride 3 x n_heads x head_dim), heads packed at their width; rotation pairs
// are (i, i + head_dim / 2) and the rope tables hold head_dim / 2 entries per
// position.  head_dim: 128 (the encoder) or 80 (the timestamp adapter).
hipError_t launch_qknorm_rope(bf16_t* qkv, const int32_t* tile_info, int n_tiles, int n_heads,
                              int head_dim, const float* qg, const float* qb, const float* kg,
                              const float* kb, const float* rope_cos, const float* rope_sin,
                              hipStream_t stream);

// out[b, p, :] = LN_f(x[s, :]) for p < P_b, else 0, with s = cu_seq[b] + p,
// or src_rows[cu_seq[b] + p] when src_rows is not NULL; bf16 output of shape
// [batch, p_max, 1280].
hipError_t launch_final_norm(const float* x, const float* g, const float* b, const int32_t* cu_seq,
                             const int32_t* src_rows, int batch, int64_t p_max, bf16_t* out,
                             hipStream_t stream);

// FP8 variant: A [M, K] and W [N, K] hold E4M3 codes (row strides lda, ldw in
// bytes, both even; K % 256 == 0, N % 128 == 0); C (op)= acc * alpha + bias
// with the epilogues above (kBiasGeluFp8 writes E4M3 codes of
// gelu(.) * out_scale, saturated at +-448); ldc counts elements of C (bytes
// for E4M3 output).
hipError_t launch_gemm_fp8(Epilogue epi, const uint8_t* A, int64_t lda, const uint8_t* W,
                           int64_t ldw, float alpha, float out_scale, const float* bias, void* C,
                           int64_t ldc, int64_t M, int N, int K, float* part, size_t part_bytes,
                           hipStream_t stream);

// Speaker fusion into the connector's operand: out[r, :] (bf16, [rows, 1280])
// = LN_f(x[s, :]) + sum_j n_j spk_tab[j, :] with s = src_rows ? src_rows[r] : r
// and n = LN_spk(act[r, :] > 0.5) over the NSPK slots (act fp32 [rows, NSPK],
// spk_tab fp32 [NSPK, 1280]).
hipError_t launch_speaker_fuse(const float* x, const float* g, const float* b,
                               const int32_t* src_rows, int64_t rows, const float* act,
                               const float* spk_g, const float* spk_b, const float* spk_tab,
                               bf16_t* out, hipStream_t stream);

// dst[r, :] = src[rows[r], :] for r < n, rows of 1024 bf16 (the stacked
// features of overlapping attention windows).
hipError_t launch_gather_rows(const bf16_t* src, const int32_t* rows, int64_t n, bf16_t* dst,
                              hipStream_t stream);

// Element conversions used when weights are copied into the context.
hipError_t launch_to_bf16(const void* src, bool src_is_bf16, bf16_t* dst, int64_t n,
                          hipStream_t stream);
hipError_t launch_to_f32(const void* src, bool src_is_bf16, float* dst, int64_t n,
                         hipStream_t stream);

// --------------------------------------------------------------- attention
// Bidirectional softmax attention per clip and head.  q, k, v are the three
// (n_heads x head_dim)-column groups of qkv [rows, 3 x n_heads x head_dim]
// (head_dim 128 for the encoder's ten heads, 80 for the timestamp adapter's
// sixteen), q and k as launch_qknorm_rope leaves them.  Work tile i
// (tile_info as for launch_qknorm_rope) covers queries [q0, min(q0 + 128,
// length)) of its sequence.  out is bf16 [rows, n_heads x head_dim] with head
// h in columns h*head_dim..., or, when out_scale > 0 (head_dim 128 only), E4M3
// codes of the output times out_scale (saturated at +-448), one byte per
// element in the same layout.
// k is read in whole 64-key tiles past a clip's end (those keys are masked),
// so qkv must have 63 readable rows after its last one.
// max_len: the longest sequence among the tiles; rows: the rows of qkv.
// With a fixed reference and long sequences whose work items would leave most
// of a last wave of workgroups idle, the keys are cut into runs whose partial
// sums go to opart / lpart (scratch of opart_bytes / lpart_bytes, free during
// the call; NULL never cuts) and are added by a second kernel.
hipError_t launch_attention(const bf16_t* qkv, const int32_t* tile_info, int n_tiles,
                            int n_heads, int head_dim, bool fixed_ref, void* out, float out_scale,
                            int max_len, int64_t rows, float* opart, size_t opart_bytes,
                            float* lpart, size_t lpart_bytes, hipStream_t stream);
// fixed_ref may be true only when |q . k| * log2(e) / sqrt(head_dim) <= 64 for
// every query and key (softmax against a fixed reference instead of a
// running maximum); attention_fixed_ref_ok decides it from the QK-norm
// parameters of a layer.
bool attention_fixed_ref_ok(const float* q_g, const float* q_b, const float* k_g,
                            const float* k_b, int dh);

}  // namespace enc
