/*
 * speech_encoder.h -- C ABI of the MI355X (gfx950) speech-encoder library
 * (libspeech_encoder.so).
 *
 * What it computes.  The page "Nemotron 3.5 Transcribe: From Recorded Speech to
 * Dataset Audits" (flozi.net), section "How audio and speakers reach the
 * language model", describes the ASR encoder branch: a 16 kHz mono waveform is
 * turned into 128 log-mel features (25 ms Hann window, 512-point FFT, 10 ms
 * hop); eight successive frames are stacked (about 100 frames/s down to 12.5
 * positions/s, 80 ms per position) and projected to width 1,280; 32
 * Transformer layers with ten heads, QK normalisation, rotary position
 * embeddings and feed-forward expansion four produce one continuous
 * 1,280-wide vector per position.  The section "How one hour fits into 65,536
 * positions" gives 12.5 positions per second; the gmlx page's Limits table
 * and the first page bound a recording at one hour.
 *
 * Where the page is silent this library reads it as follows (the CPU oracle
 * used by the tests makes the same choices): frame t = samples
 * [160 t, 160 t + 400), F = 1 + floor((N - 400) / 160) frames (0 if N < 400);
 * periodic Hann window; power spectrum |X_k|^2, k = 0..256; Slaney mel bank
 * with peak-1 triangles; natural log of (energy + 2^-24); P = ceil(F / 8)
 * positions with frame-major stacking and zero tail frames; linear maps with
 * bias in the [out, in] layout; pre-norm blocks with a final LayerNorm;
 * LayerNorm with biased variance and eps 1e-5; QK-norm = LayerNorm over each
 * head's 128 dims (gain/bias shared by heads), before rotation; rotation of
 * pairs (i, i + 64) by p * 10000^(-i/64); bidirectional attention over the
 * whole clip; FFN 1280 -> 5120 -> 1280 with exact-erf GELU.
 *
 * Precision.  GEMM and attention operands are bf16 with fp32 accumulation;
 * the residual stream, norm statistics, softmax and rotation run in fp32; the
 * frontend's window, transform, power and mel sums run in float64 and its log
 * is rounded to fp32.
 *
 * Conventions for every call below.
 *   - Device pointers are HIP device memory on the current device; host
 *     pointers are ordinary host memory.  "stream" is a hipStream_t on which
 *     all device work of the call is enqueued; calls return without waiting
 *     for that work (except enc_create, which is synchronous).
 *   - Every argument and size check happens before anything is enqueued: a
 *     call that returns an error has not written any output.
 *   - A return value other than ENC_OK leaves a message for
 *     enc_last_error() (per thread).  No C++ exception crosses the ABI.
 *   - One context serves one stream / host thread at a time.
 */
#ifndef SPEECH_ENCODER_H
#define SPEECH_ENCODER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ENC_ABI_VERSION 1

/* Status codes. */
#define ENC_OK 0
#define ENC_ERR_ARG 1       /* NULL pointer, bad version, batch < 1, length < 0 ... */
#define ENC_ERR_TOO_LONG 2  /* a clip longer than one hour (57,600,000 samples)      */
#define ENC_ERR_NOMEM 3     /* device memory (or the workspace cap) does not fit     */
#define ENC_ERR_HIP 4       /* a HIP runtime call or kernel launch failed            */

/* Element type of the weight tensors handed to enc_create. */
#define ENC_F32 0
#define ENC_BF16 1

/* Model constants. */
#define ENC_D_MODEL 1280
#define ENC_N_HEADS 10
#define ENC_HEAD_DIM 128
#define ENC_FFN_DIM 5120
#define ENC_N_MELS 128
#define ENC_STACK 8
#define ENC_MAX_SAMPLES 57600000LL

/* One Transformer layer: DEVICE pointers, element type enc_weights.dtype,
 * linear weights row-major [out, in]. */
typedef struct enc_layer_weights {
  const void* ln1_g;   /* [1280]        pre-attention LayerNorm gain          */
  const void* ln1_b;   /* [1280]        and bias                              */
  const void* w_qkv;   /* [3840, 1280]  rows 0..1279 Q, 1280..2559 K, rest V  */
  const void* b_qkv;   /* [3840]                                              */
  const void* q_g;     /* [128]         QK-norm gain/bias for q (all heads)   */
  const void* q_b;     /* [128]                                               */
  const void* k_g;     /* [128]         QK-norm gain/bias for k (all heads)   */
  const void* k_b;     /* [128]                                               */
  const void* w_o;     /* [1280, 1280]  attention output projection           */
  const void* b_o;     /* [1280]                                              */
  const void* ln2_g;   /* [1280]        pre-FFN LayerNorm                     */
  const void* ln2_b;   /* [1280]                                              */
  const void* w_up;    /* [5120, 1280]  FFN expansion                         */
  const void* b_up;    /* [5120]                                              */
  const void* w_down;  /* [1280, 5120]  FFN contraction                       */
  const void* b_down;  /* [1280]                                              */
} enc_layer_weights;

typedef struct enc_weights {
  int32_t abi_version;              /* must be ENC_ABI_VERSION                 */
  int32_t n_layers;                 /* >= 1 (32 for the full encoder)          */
  int32_t dtype;                    /* ENC_F32 or ENC_BF16, for every tensor   */
  int32_t reserved;                 /* 0                                       */
  const void* w_in;                 /* [1280, 1024] stacked-frame projection   */
  const void* b_in;                 /* [1280]                                  */
  const enc_layer_weights* layers;  /* HOST array of n_layers entries          */
  const void* lnf_g;                /* [1280] final LayerNorm                  */
  const void* lnf_b;                /* [1280]                                  */
} enc_weights;

typedef struct enc_ctx enc_ctx;

/*
 * enc_create: copy the weights into a new context.
 *   w    host struct describing device tensors (see enc_weights).  Matrices
 *        are converted to bf16 (round to nearest even) and biases/gains to
 *        fp32 in context-owned device memory; the caller may free its tensors
 *        once the call returns.  The context also builds its constant tables
 *        on the host in float64 (window, FFT twiddles and mel bank, kept in
 *        float64; rotation cos/sin, rounded once to fp32) and allocates its
 *        fixed scratch (split-K partial sums, 64 MiB).
 *   out  receives the handle (host pointer).
 * Synchronous.  Errors: ENC_ERR_ARG (NULL, wrong abi_version, n_layers < 1,
 * unknown dtype, NULL tensor), ENC_ERR_NOMEM, ENC_ERR_HIP.
 */
int enc_create(const enc_weights* w, enc_ctx** out);

/*
 * enc_logmel: log-mel features of a batch of clips (frontend only).
 *   audio    DEVICE fp32 [batch, N_max], row-major, N_max = max(lengths);
 *            clip b is audio[b, 0 : lengths[b]], the rest is ignored.
 *   lengths  HOST int64 [batch], samples per clip, 0 <= lengths[b] <= 57,600,000.
 *   out      DEVICE fp32 [batch, F_max, 128], F_max = F(N_max); frames
 *            t >= F(lengths[b]) are written as 0.0.
 * Errors: ENC_ERR_ARG (NULL, batch < 1, negative length), ENC_ERR_TOO_LONG,
 * ENC_ERR_HIP.  audio may be NULL only if N_max == 0.
 */
int enc_logmel(enc_ctx* ctx, const float* audio, const int64_t* lengths, int32_t batch,
               float* out, hipStream_t stream);

/*
 * enc_forward: the whole encoder, waveform to embeddings.
 *   audio, lengths as for enc_logmel.
 *   out_embeddings  DEVICE bf16 [batch, P_max, 1280], P_max = ceil(F_max / 8);
 *            row p of clip b is its position-p embedding for p < P_b =
 *            ceil(F(lengths[b]) / 8) and 0 otherwise.  Each clip is encoded
 *            as its own sequence: attention and norms never mix clips, and
 *            padding never reaches a clip.  The batch's total length does
 *            choose how the matrix products split their last round of tiles,
 *            so a clip's rows may differ from a run of that clip alone by
 *            fp32 summation order (rounding); repeating a call with the same
 *            batch gives bit-identical output.
 * The context keeps a workspace sized by the batch's total positions; a call
 * that needs a larger one first waits for the stream, then reallocates.  The
 * environment variable ENC_WORKSPACE_CAP_BYTES, read at each call, caps the
 * workspace: a call that would need more returns ENC_ERR_NOMEM, as does one
 * whose allocation fails.  Errors: as enc_logmel, plus ENC_ERR_NOMEM.
 */
int enc_forward(enc_ctx* ctx, const float* audio, const int64_t* lengths, int32_t batch,
                void* out_embeddings, hipStream_t stream);

/*
 * enc_forward_noalloc: enc_forward for callers that cannot allocate device
 * memory during the call -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, output and
 * results as enc_forward (same kernels, bit-identical embeddings), but every
 * per-call device buffer (workspace, plan arrays, split-K partial sums) comes
 * from one static device array of ENC_NOALLOC_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends; the call allocates
 * nothing and frees nothing (the context's pinned plan staging is made by
 * enc_create).
 *   Limit: the workspace must fit ENC_NOALLOC_SCRATCH_BYTES minus 66 MiB
 *   (about 7,000 positions in one call, i.e. roughly nine minutes of audio;
 *   enc_workspace_bytes reports a batch's need); larger batches return
 *   ENC_ERR_NOMEM before anything is enqueued.
 *   Sharing: every enc_forward_noalloc call on a GPU, from any context or
 *   thread, uses that GPU's one array, which keeps the last call's contents.
 *   Calls that overlap on one GPU (different streams, or no ordering between
 *   them) race and give undefined results; serialize them.  No part of the
 *   array needs to start at zero: each call writes every element it reads.
 *   Kernel timing brackets (enc_profile_kernel) do not apply to this call.
 * Errors: as enc_forward (ENC_ERR_NOMEM when the batch exceeds the limit;
 * ENC_ERR_HIP if the array's device address could not be obtained).
 */
#define ENC_NOALLOC_SCRATCH_BYTES (256u << 20)
int enc_forward_noalloc(enc_ctx* ctx, const float* audio, const int64_t* lengths, int32_t batch,
                        void* out_embeddings, hipStream_t stream);

/*
 * enc_set_attention: the attention scope of later enc_forward calls on ctx.
 * The pages describe the encoder as trained on 30-second chunks and served
 * with local windows (500 positions of core plus 50 of context on each side,
 * "Local encoder windows, recording-wide language context"); this call
 * selects between full-clip attention and such windows.
 *   mode ENC_ATTN_FULL (default): each clip is one sequence; core and
 *        context must be 0.
 *   mode ENC_ATTN_WINDOWS: position p of a clip with P positions belongs to
 *        window w = floor(p / core).  Window w is encoded as an independent
 *        input: its sequence is positions [max(0, w*core - context),
 *        min(P, (w+1)*core + context)) of the clip's stacked features, with
 *        attention only inside it and rotary positions counted from its
 *        first position; position p's embedding is the one computed in its own
 *        window (context positions are computed and discarded).  context = 0
 *        gives non-overlapping chunks (core = 375 is the pages' 30 seconds);
 *        core = 500, context = 50 gives the serving windows.
 *        Requires core >= 1, context >= 0, core + 2*context <= 45,000.
 * The output layout is unchanged.  Windows with context duplicate the context
 * rows, so the workspace grows by their share (enc_workspace_bytes reports
 * the full-attention size).  Host-only; errors: ENC_ERR_ARG.
 */
#define ENC_ATTN_FULL 0
#define ENC_ATTN_WINDOWS 1
int enc_set_attention(enc_ctx* ctx, int32_t mode, int32_t core, int32_t context);

/*
 * Speaker fusion and identity connector.  The page's section "How audio and
 * speakers reach the language model" adds speaker activity to the ASR
 * states before the language model: activity of up to eight speaker slots,
 * aligned to the encoder's 80 ms grid, is thresholded at 0.5, normalised by a
 * learned LayerNorm over the slots and mapped to width 1,280 by a fixed
 * sinusoidal speaker kernel (saved scale 1); the sum keeps the positions and
 * the width.  One learned linear map (no temporal downsampling) then takes
 * the fused states to the language model's width (2,688 in the section "What
 * the 52 backbone blocks actually do").  The formulas did not survive the
 * page's extraction; this library reads them as:
 *   b    = [a > 0.5] per slot (a = activity probability, fp32 compare)
 *   n    = LayerNorm(b) over the 8 slots (biased variance, eps 1e-5, gain, bias)
 *   K    = scale * [sin(s w_i), cos(s w_i)] interleaved over columns 2i, 2i+1,
 *          s = slot index 0..7, w_i = 10000^(-2i/1280) (the sinusoid table of
 *          the original Transformer with the slot index as position)
 *   fused = H + n K,   z = fused W_c^T + b_c
 * with H the encoder output (final LayerNorm included).
 */
#define ENC_SPEAKERS 8
#define ENC_LLM_DIM 2688

typedef struct enc_connector_weights {
  int32_t abi_version;    /* must be ENC_ABI_VERSION                          */
  int32_t dtype;          /* ENC_F32 or ENC_BF16, for every tensor            */
  int32_t out_dim;        /* language-model width: a multiple of 128, 128..65536 */
  float speaker_scale;    /* scale of the fixed speaker kernel (1 in the release) */
  const void* spk_ln_g;   /* DEVICE [8]            speaker LayerNorm gain      */
  const void* spk_ln_b;   /* DEVICE [8]            and bias                    */
  const void* w_conn;     /* DEVICE [out_dim, 1280] connector weight          */
  const void* b_conn;     /* DEVICE [out_dim]       connector bias            */
} enc_connector_weights;

/*
 * enc_set_connector: copy speaker-fusion and connector weights into ctx
 * (w_conn to bf16, the rest to fp32; the kernel table is built on the host in
 * float64 and rounded once to fp32), replacing any earlier set.  Synchronous.
 * Errors: ENC_ERR_ARG (NULL, wrong abi_version, unknown dtype, bad out_dim,
 * non-finite scale), ENC_ERR_NOMEM, ENC_ERR_HIP.
 */
int enc_set_connector(enc_ctx* ctx, const enc_connector_weights* w);

/*
 * enc_forward_fused: waveform and speaker activity to language-model input
 * rows: the encoder as in enc_forward (same attention scope), then speaker
 * fusion and the connector.
 *   audio, lengths  as for enc_logmel.
 *   activity  DEVICE fp32 [R, 8], R = sum_b P_b: the rows of clip b are
 *             R_b = sum_{b' < b} P_b' .. R_b + P_b - 1 (clips packed in order,
 *             no padding), row R_b + p holds the activity of the 8 slots at
 *             position p (80 ms grid).
 *   out       DEVICE bf16 [R, out_dim], packed the same way.
 * Requires an earlier enc_set_connector.  Errors: as enc_forward, and
 * ENC_ERR_ARG when no connector is set or activity/out is NULL with R > 0.
 * R = 0 (every clip shorter than 400 samples) writes nothing.
 */
int enc_forward_fused(enc_ctx* ctx, const float* audio, const int64_t* lengths, int32_t batch,
                      const float* activity, void* out, hipStream_t stream);

/*
 * FP8 variant.  The nemotron-transcribe skill page, section "Precision
 * selection", describes an FP8 release (a ModelOpt export) with a quantized
 * audio encoder; the Dataset Audits page, section "The long-audio memory
 * budget is not just the KV cache", keeps the ASR projections in FP8.  This
 * library reads that as the per-tensor FP8 scheme:
 *   - the four linear maps of every layer (QKV, attention output, FFN up,
 *     FFN down) multiply E4M3 codes (OCP FP8, largest value 448) with fp32
 *     accumulation: y = (q_x . q_w) * fp32(s_x * s_w) + b;
 *   - weight codes q_w = e4m3(sat(w * fp32(1 / s_w))), s_w = amax|w| / 448,
 *     from the context's bf16 copy of each matrix (s_w = 1 for a zero matrix);
 *   - input codes q_x = e4m3(sat(x * fp32(1 / s_x))) with one static scale s_x
 *     per linear map (a calibration result: amax / 448 over calibration data);
 *     the producers (LayerNorm, attention, the FFN's GELU) write the codes;
 *   - the input projection, attention, the norms and the connector stay as in
 *     the bf16 encoder.
 * e4m3() rounds to nearest even; sat() clamps to [-448, 448].
 */
#define ENC_PREC_BF16 0
#define ENC_PREC_FP8 1

/*
 * enc_set_precision: the precision of later enc_forward(_fused) calls.
 *   ENC_PREC_BF16 (default): input_scales is ignored (may be NULL).
 *   ENC_PREC_FP8: input_scales is a HOST float array [n_layers][4], the input
 *   scales s_x of (QKV, attention output, FFN up, FFN down) of each layer,
 *   each positive and finite.  The first FP8 call quantizes the weights
 *   (synchronous; 631 MB of codes for 32 layers kept in the context).
 * Errors: ENC_ERR_ARG, ENC_ERR_NOMEM, ENC_ERR_HIP.
 */
int enc_set_precision(enc_ctx* ctx, int32_t precision, const float* input_scales);

/*
 * enc_calibrate: run the bf16 encoder on a batch (as enc_forward, same
 * attention scope, no output) and return in amax (HOST float [n_layers][4])
 * the largest magnitude of the input of each quantizable linear map: the
 * LayerNorm outputs feeding QKV and FFN up, the attention output and the
 * GELU output, as the bf16 values those maps read.  Synchronous.  Input
 * scales for enc_set_precision are amax / 448 (merge several batches by
 * taking the maximum).  Errors: as enc_forward.
 */
int enc_calibrate(enc_ctx* ctx, const float* audio, const int64_t* lengths, int32_t batch,
                  float* amax, hipStream_t stream);

/*
 * enc_fp8_input_scales: host-only.  The input scales enc_set_precision takes,
 * from the amax values enc_calibrate returns (merged over batches by the
 * caller): scales[i] = amax[i] / 448 in fp32, or 1 where amax[i] is 0 (a map
 * whose input was all zero).  n = n_layers * 4.  Errors: ENC_ERR_ARG (NULL
 * with n > 0, n < 0, an amax that is negative or not finite).
 */
int enc_fp8_input_scales(const float* amax, int32_t n, float* scales);

/*
 * CTC timestamp adapter.  The Dataset Audits page, section "4. Use alignment
 * and audio questions as supporting evidence", describes a ~50M-parameter
 * adapter on the unfused ASR states (width 1,280, 80 ms grid): a stride-two
 * transposed convolution to a 40 ms grid, two Transformer layers with 16
 * heads, and a projection to 23,862 tokens plus the CTC blank, whose frame
 * probabilities forced alignment consumes.  This library reads it as:
 *   - input: the encoder output (final LayerNorm included, before fusion);
 *   - upsampling: kernel 2, stride 2: frame 2t + j = H[t] W_j^T + b_conv;
 *   - layers: the encoder's block type with 16 heads of width 80 (QK-norm
 *     over 80 dims, rotation of pairs (i, i + 40) at the frame's position on
 *     the 40 ms grid, bidirectional attention over the whole clip) and a
 *     feed-forward width of 1,280 (53.5M parameters in all, the stated ~50M);
 *   - a final LayerNorm, the projection, log-softmax over the classes.
 */
typedef struct enc_ctc_weights {
  int32_t abi_version;              /* must be ENC_ABI_VERSION                   */
  int32_t dtype;                    /* ENC_F32 or ENC_BF16, for every tensor     */
  int32_t n_layers;                 /* 1..8 (2 in the release)                   */
  int32_t n_classes;                /* 2..1048576 (23,863: 23,862 tokens + blank) */
  const void* w_conv;               /* DEVICE [2, 1280, 1280]: tap j, [out, in]  */
  const void* b_conv;               /* DEVICE [1280]                             */
  const enc_layer_weights* layers;  /* HOST array [n_layers] of DEVICE tensors with
                                       head width 80: q_g, q_b, k_g, k_b [80];
                                       w_qkv [3840, 1280] (head h of q/k/v in rows
                                       80 h ..); w_o, w_up, w_down [1280, 1280];
                                       b_up [1280]; the rest as for the encoder */
  const void* lnf_g;                /* DEVICE [1280] final LayerNorm              */
  const void* lnf_b;                /* DEVICE [1280]                             */
  const void* w_out;                /* DEVICE [n_classes, 1280]                  */
  const void* b_out;                /* DEVICE [n_classes]                        */
} enc_ctc_weights;

/*
 * enc_set_ctc: copy adapter weights into ctx (matrices to bf16, vectors to
 * fp32, q/k/v heads into 128-wide slots whose extra dims are zero), replacing
 * any earlier set.  Synchronous.  Errors: ENC_ERR_ARG, ENC_ERR_NOMEM,
 * ENC_ERR_HIP.
 */
int enc_set_ctc(enc_ctx* ctx, const enc_ctc_weights* w);

/*
 * enc_forward_ctc: waveform to CTC log-probabilities: the encoder as in
 * enc_forward (same attention scope and precision), then the adapter (its
 * attention always over the whole clip).
 *   audio, lengths  as for enc_logmel.
 *   out_logprobs  DEVICE fp32 [2 R, n_classes], R = sum_b P_b: clip b's frames
 *                 are rows 2 R_b .. 2 R_b + 2 P_b - 1 (R_b = sum_{b' < b} P_b'),
 *                 frame f at f x 40 ms; each row is log-probabilities over the
 *                 classes (blank last, as the weights order them).
 * The adapter keeps its own workspace (about 250 KB per encoder position,
 * most of it the padded logits).  Requires an earlier enc_set_ctc.  Errors: as
 * enc_forward, and ENC_ERR_ARG without adapter weights or with a NULL output
 * and R > 0.  R = 0 writes nothing.
 */
int enc_forward_ctc(enc_ctx* ctx, const float* audio, const int64_t* lengths, int32_t batch,
                    float* out_logprobs, hipStream_t stream);

/*
 * enc_ctc_align: CTC forced alignment of given token sequences onto CTC
 * log-probabilities -- the step that turns the adapter's frame
 * probabilities and a generated transcript into token timestamps
 * ("Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
 * section "4. Use alignment and audio questions as supporting evidence").
 * Per clip, the most probable CTC path that spells the tokens (Viterbi over
 * blank, y1, blank, ..., yL, blank; a blank separates equal neighbours),
 * decided in float32; ties go to staying in a state, then to the nearer
 * predecessor, and at the end to the final blank.
 *   log_probs  DEVICE fp32, clip-packed rows [sum_b frames[b], ld]: clip b's
 *              rows follow the earlier clips' (enc_forward_ctc's output, with
 *              frames[b] = 2 P_b and ld = n_classes); class n_classes - 1 is
 *              the blank.  Any finite scores work (they need not be
 *              normalised).
 *   frames     HOST int64 [batch], >= 0.
 *   tokens     HOST int32, every clip's token ids concatenated, each in
 *              0 .. n_classes - 2 (NULL if there are none).
 *   n_tokens   HOST int64 [batch], >= 0, at most 1,023 per clip.
 *   spans      DEVICE int32 [sum_b n_tokens[b], 2]: first and last frame the
 *              path spends on each token (frame f at f x 40 ms on the
 *              adapter's grid); -1, -1 for a clip without alignment.
 *   scores     DEVICE fp32 [batch]: the best path's log-probability; -inf
 *              when the tokens cannot fit the frames (fewer frames than
 *              tokens plus equal neighbours) -- a review signal, not an error.
 * Runs on `stream` on the context's device; the context keeps a workspace of
 * about sum_b frames[b] x (2 n_tokens[b] + 1) bytes, grown as needed (calls
 * on one context must not overlap).  Errors: ENC_ERR_ARG (NULL pointers,
 * ld < n_classes, negative counts, a token outside the vocabulary),
 * ENC_ERR_TOO_LONG (more than 1,023 tokens in a clip), ENC_ERR_NOMEM,
 * ENC_ERR_HIP; nothing is launched then.
 */
int enc_ctc_align(enc_ctx* ctx, const float* log_probs, int64_t ld, int32_t n_classes,
                  const int64_t* frames, const int32_t* tokens, const int64_t* n_tokens,
                  int32_t batch, int32_t* spans, float* scores, hipStream_t stream);

/* enc_destroy: wait for the context's device work and free it.  NULL is a
 * no-op. */
void enc_destroy(enc_ctx* ctx);

/*
 * enc_shapes: host-only.  F_max and P_max (HOST int64 out-pointers) of a
 * batch.  Errors: ENC_ERR_ARG, ENC_ERR_TOO_LONG.
 */
int enc_shapes(const int64_t* lengths, int32_t batch, int64_t* f_max, int64_t* p_max);

/*
 * enc_workspace_bytes: host-only.  Device bytes enc_forward's workspace needs
 * for this batch with full-clip attention (independent of n_layers >= 1).
 * Errors: ENC_ERR_ARG, ENC_ERR_TOO_LONG.
 */
int enc_workspace_bytes(int32_t n_layers, const int64_t* lengths, int32_t batch, size_t* bytes);

/* enc_last_error: message of this thread's last failed call ("" if none). */
const char* enc_last_error(void);

/*
 * Kernel timing for measurement.  enc_profile_kernel(ctx, id) brackets every
 * launch of kernel class id (ENC_K_*) made by later enc_forward(_fused) calls with a
 * pair of HIP events on the call's stream; id = -1 turns this off.
 * enc_profile_read(ctx, &launches, &total_ms) waits for those events and
 * returns the number of bracketed launches and their summed duration, then
 * clears the record.  Errors: ENC_ERR_ARG, ENC_ERR_HIP.
 */
#define ENC_K_FRONTEND 0
#define ENC_K_GEMM_IN 1
#define ENC_K_LAYERNORM 2
#define ENC_K_GEMM_QKV 3
#define ENC_K_QKNORM_ROPE 4
#define ENC_K_ATTENTION 5
#define ENC_K_GEMM_O 6
#define ENC_K_GEMM_UP 7
#define ENC_K_GEMM_DOWN 8
#define ENC_K_FINAL_NORM 9
#define ENC_K_SPEAKER_FUSE 10   /* enc_forward_fused: final norm + speaker fusion */
#define ENC_K_CONNECTOR 11      /* enc_forward_fused: connector GEMM              */
#define ENC_K_CTC 12            /* enc_forward_ctc: upsampling and adapter layers */
#define ENC_K_CTC_OUT 13        /* enc_forward_ctc: final norm, projection, log-softmax */
#define ENC_K_COUNT 14
int enc_profile_kernel(enc_ctx* ctx, int32_t kernel_id);
int enc_profile_read(enc_ctx* ctx, int64_t* launches, double* total_ms);

/*
 * enc_probe_peaks: what this device sustains, measured, as context for the
 * roofline fractions of the encoder's kernels (the published MI355X peaks,
 * 2.5 PFLOP/s dense bf16 and 8 TB/s, assume the peak clock and ideal DRAM
 * efficiency).  Not part of the encoder.
 *   (a) a register-only kernel of back-to-back dense bf16 MFMAs
 *       (v_mfma_f32_32x32x16_bf16, eight independent accumulators per
 *       wavefront, two wavefronts per SIMD on every CU) -> *mfma_tflops,
 *       dense bf16 TFLOP/s;
 *   (b) a device copy of `bytes` bytes from src to dst, 16 bytes per lane
 *       -> *copy_gbs, bytes read plus bytes written per second, in GB/s.
 * Each runs once untimed, then `reps` times between two HIP events on
 * `stream` (NULL: the default stream); the call waits for them.
 * dst, src: caller-owned device buffers of `bytes` bytes, bytes % 16 == 0,
 * bytes >= 1 MiB; dst's contents are overwritten (it also receives the MFMA
 * kernel's sums).  reps >= 1.  Errors: ENC_ERR_ARG, ENC_ERR_HIP.
 */
int enc_probe_peaks(void* dst, const void* src, size_t bytes, int32_t reps, void* stream,
                    double* mfma_tflops, double* copy_gbs);

#ifdef __cplusplus
}
#endif

#endif /* SPEECH_ENCODER_H */
