// CTC forced alignment (align.hip): the launcher's interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace enc {

// CTC forced alignment (align.hip): one clip per workgroup.  Clip b's
// log-probabilities are rows row0 .. row0 + frames - 1 of lp (row stride ld,
// blank = class `blank`); its tokens are tokens[tok_off .. tok_off + n_tok);
// its per-frame choices take frames x (2 n_tok + 1) bytes of `back` from
// back_off.  Writes spans[2 (tok_off + i)], [.. + 1] = first and last frame of
// token i (-1 when the clip has no alignment) and scores[b] (the best path's
// log-probability, -inf when none).  2 n_tok + 1 <= ALIGN_MAX_STATES.
struct AlignClip {
  int64_t row0;
  int64_t back_off;
  int32_t frames;
  int32_t tok_off;
  int32_t n_tok;
  int32_t pad;
};
constexpr int ALIGN_MAX_STATES = 2048;
hipError_t launch_ctc_align(const float* lp, int64_t ld, int blank, const AlignClip* clips,
                            int batch, const int32_t* tokens, uint8_t* back, int32_t* spans,
                            float* scores, int max_states, hipStream_t stream);

}  // namespace enc
