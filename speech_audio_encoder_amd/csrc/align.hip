// CTC forced alignment of a given token sequence on gfx950.
//
// Method: after decoding, the generated word sequence is forced onto the CTC
// adapter's frame probabilities (40 ms grid), which gives the word
// timestamps ("Nemotron 3.5 Transcribe: From Recorded Speech to Dataset
// Audits", section "4. Use alignment and audio questions as supporting
// evidence").  The alignment is the most probable CTC path that spells the
// tokens (Viterbi): states s = 0 .. 2L of the sequence blank, y1, blank, ...,
// yL, blank; a path starts in state 0 or 1, ends in 2L or 2L - 1, and moves
// from s to s, s + 1, or s + 2 when state s + 2 holds a token that differs
// from the one in state s.  Scores are float32 sums of the frames'
// log-probabilities, taken frame by frame; ties between predecessors go to
// the state that stays, then s - 1, then s - 2, and between the final
// states to the blank.
//
// Work split: one workgroup of four wavefronts per clip.  The recursion over
// frames is sequential; within a frame every state is independent, so thread
// i owns states i, i + 256, ... (SPT of them) and the scores of the previous
// frame live in LDS (two buffers, one barrier per frame).  The choices of 32
// frames gather in LDS before they are copied out together.  The
// log-probabilities a thread needs are gathered DEPTH frames ahead into
// registers, so the per-frame chain does not wait on global memory.  Each
// frame's choices (0, 1, 2: how far back the best predecessor lies) are
// written as bytes; thread 0 then walks them back from the final state,
// 64 frames at a time out of an LDS window that the workgroup loads (the
// path moves at most two states per frame), and writes each token's first
// and last frame.

#include <cmath>

#include "common.h"
#include "align.h"

namespace enc {

namespace {

constexpr int AT = 256;          // threads per workgroup (four wavefronts)
constexpr int WALK = 64;         // frames per backtracking window
constexpr int WIN_W = 2 * WALK + 1;   // states a window can span
constexpr int CHUNK = 32;        // frames whose choices are gathered in LDS before a copy out

// SPT states per thread, log-probabilities prefetched DEPTH frames ahead.
template <int SPT, int DEPTH>
__global__ __launch_bounds__(AT) void ctc_align_kernel(const float* __restrict__ lp, int64_t ld,
                                                       int blank, const AlignClip* __restrict__ clips,
                                                       const int32_t* __restrict__ tokens,
                                                       uint8_t* __restrict__ back,
                                                       int32_t* __restrict__ spans,
                                                       float* __restrict__ scores) {
  __shared__ float dp[2][AT * SPT];
  __shared__ uint8_t win[WALK][WIN_W + 3];
  __shared__ uint8_t chunk[CHUNK * AT * SPT];   // choices of up to CHUNK frames, [frame][state]
  __shared__ int s_rep;

  const int tid = threadIdx.x;
  const AlignClip c = clips[blockIdx.x];
  const int T = c.frames, L = c.n_tok, S = 2 * L + 1;
  const int32_t* tok = tokens + c.tok_off;

  // equal neighbours (each needs a blank between them)
  if (tid == 0) s_rep = 0;
  __syncthreads();
  int rep = 0;
  for (int i = tid + 1; i < L; i += AT) rep += tok[i] == tok[i - 1];
  if (rep) atomicAdd(&s_rep, rep);
  __syncthreads();
  if (T < max(1, L + s_rep)) {   // no alignment
    for (int i = tid; i < L; i += AT) {
      spans[2 * (c.tok_off + i)] = -1;
      spans[2 * (c.tok_off + i) + 1] = -1;
    }
    if (tid == 0) scores[blockIdx.x] = -INFINITY;
    return;
  }

  // this thread's states: class and whether s - 2 may precede them
  int lab[SPT];
  bool skip[SPT], live[SPT];
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int s = tid + AT * k;
    live[k] = s < S;
    lab[k] = blank;
    skip[k] = false;
    if (live[k] && (s & 1)) {   // token (s - 1) / 2 < L
      const int i = (s - 1) >> 1;
      lab[k] = tok[i];
      if (i >= 1) skip[k] = tok[i] != tok[i - 1];
    }
  }
  const float* base = lp + c.row0 * ld;
  uint8_t* bk = back + c.back_off;

  // frame 0
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int s = tid + AT * k;
    if (live[k]) dp[0][s] = s <= 1 ? base[lab[k]] : -INFINITY;
  }
  // log-probabilities of frames 1 .. DEPTH
  float pre[DEPTH][SPT];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
#pragma unroll
    for (int k = 0; k < SPT; ++k) pre[d][k] = base[(int64_t)min(1 + d, T - 1) * ld + lab[k]];
  __syncthreads();

  // Frames t = t0 + d (d = 0 .. DEPTH-1), t0 = 1, 1 + DEPTH, ...  The
  // choices of CHUNK frames gather in LDS and are then copied out together:
  // a global store inside the per-frame chain would make every frame wait
  // for all outstanding loads (loads and stores share one counter and may
  // complete out of order), the prefetched log-probabilities included.
  static_assert(CHUNK % DEPTH == 0, "chunk of whole prefetch rounds");
  for (int c0 = 1; c0 < T; c0 += CHUNK) {
    for (int t0 = c0; t0 < c0 + CHUNK && t0 < T; t0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int t = t0 + d;
        const bool act = t < T;   // the last round's frames past T only keep the pattern
        const float* prv = dp[(t - 1) & 1];
        float* cur = dp[t & 1];
        uint8_t* ch = chunk + (t - c0) * S;
        // (every lane computes and loads in every frame of the round --
        // states past S read in-bounds LDS and the blank's column, frames
        // past T reload the last row -- so that no load sits in a branch and
        // each frame waits only for the load made DEPTH frames earlier; only
        // live states of frames before T are stored)
        const int tn = min(t + DEPTH, T - 1);   // past the end: a spare in-bounds load
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
          const int s = tid + AT * k;
          float best = prv[s];
          uint8_t bp = 0;
          const float m1 = s >= 1 ? prv[max(s - 1, 0)] : -INFINITY;
          if (m1 > best) {
            best = m1;
            bp = 1;
          }
          const float m2 = skip[k] ? prv[max(s - 2, 0)] : -INFINITY;
          if (m2 > best) {
            best = m2;
            bp = 2;
          }
          const float v = pre[d][k] + best;
          if (act && live[k]) {
            cur[s] = v;
            ch[s] = bp;
          }
          // the same register, DEPTH frames later
          pre[d][k] = base[(int64_t)tn * ld + lab[k]];
        }
        // LDS only: the scores and choices of this frame are written
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
    // copy the chunk's choices (frames c0 .. c0 + rows - 1, contiguous in
    // both places) out; the barrier lets the next chunk reuse the buffer
    const int bytes = min(CHUNK, T - c0) * S;
    uint8_t* dst = bk + (int64_t)c0 * S;
    for (int e = tid; e < bytes; e += AT) dst[e] = chunk[e];
    // wait here, once per chunk, for the stores (and every prefetch in
    // flight), so that within a chunk only loads are outstanding and each
    // frame waits just for its own log-probabilities
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // final state (ties to the blank), score
  const float* fin = dp[(T - 1) & 1];
  int s = S - 1;
  if (S > 1 && fin[S - 2] > fin[S - 1]) s = S - 2;
  const float score = fin[s];
  if (!(score > -INFINITY)) {   // only -inf log-probabilities reach here
    for (int i = tid; i < L; i += AT) {
      spans[2 * (c.tok_off + i)] = -1;
      spans[2 * (c.tok_off + i) + 1] = -1;
    }
    if (tid == 0) scores[blockIdx.x] = -INFINITY;
    return;
  }
  if (tid == 0) scores[blockIdx.x] = score;

  // Walk back WALK frames at a time: frames t_lo .. t_hi and states
  // max(0, s - 2 WALK) .. s (the path moves at most two states a frame) are
  // loaded into LDS by the workgroup, then followed by thread 0, which
  // records each token's last frame when it first meets the token's state
  // and its first frame when it leaves it.  The walk's state at t_hi and at
  // t_hi + 1 pass from window to window through LDS.
  __shared__ int s_state, s_after;
  if (tid == 0) {
    s_state = s;
    s_after = -1;   // no frame after the last one
  }
  __syncthreads();
  for (int t_hi = T - 1; t_hi >= 0; t_hi -= WALK) {
    const int t_lo = max(0, t_hi - WALK + 1);
    const int s_hi = s_state;
    const int s_lo = max(0, s_hi - 2 * WALK);
    const int w = s_hi - s_lo + 1;
    for (int e = tid; e < (t_hi - t_lo + 1) * w; e += AT) {
      const int r = e / w, q = e - r * w;
      win[r][q] = bk[(int64_t)(t_lo + r) * S + s_lo + q];
    }
    __syncthreads();
    if (tid == 0) {
      int st = s_hi, after = s_after;
      for (int t = t_hi; t >= t_lo; --t) {
        if (st & 1) {   // token (st - 1) / 2
          const int i = c.tok_off + ((st - 1) >> 1);
          if (st != after) spans[2 * i + 1] = t;   // its last frame
          spans[2 * i] = t;                        // its first frame, so far
        }
        after = st;
        if (t > 0) st -= win[t - t_lo][st - s_lo];   // frame 0 has no predecessor
      }
      s_state = st;
      s_after = after;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_ctc_align(const float* lp, int64_t ld, int blank, const AlignClip* clips,
                            int batch, const int32_t* tokens, uint8_t* back, int32_t* spans,
                            float* scores, int max_states, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (batch < 0 || max_states < 1 || max_states > ALIGN_MAX_STATES || blank < 0)
    return hipErrorInvalidValue;
  const dim3 grid(batch), block(AT);
  if (max_states <= AT)
    ctc_align_kernel<1, 16><<<grid, block, 0, stream>>>(lp, ld, blank, clips, tokens, back, spans,
                                                        scores);
  else if (max_states <= 2 * AT)
    ctc_align_kernel<2, 8><<<grid, block, 0, stream>>>(lp, ld, blank, clips, tokens, back, spans,
                                                       scores);
  else if (max_states <= 4 * AT)
    ctc_align_kernel<4, 4><<<grid, block, 0, stream>>>(lp, ld, blank, clips, tokens, back, spans,
                                                       scores);
  else
    ctc_align_kernel<8, 4><<<grid, block, 0, stream>>>(lp, ld, blank, clips, tokens, back, spans,
                                                       scores);
  return hipGetLastError();
}

}  // namespace enc
