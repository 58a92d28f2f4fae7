"""CTC forced alignment on the GPU (enc_ctc_align) against the oracle.

"Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
"4. Use alignment and audio questions as supporting evidence".  Both sides
take every decision in float32 with the same tie rules, so scores must match
bit for bit and spans exactly.  Inputs are seeded synthetic frame scores
(workloads.alignment_case); none comes from the GPU path.
"""

import numpy as np
import pytest

import oracle
from oracle import align
from speech_audio_encoder_amd import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def enc():
    import torch  # noqa: F401
    from speech_audio_encoder_amd import binding
    e = binding.Encoder(workloads.workload_weights("tiny"), dtype="f32")
    yield e
    e.close()


def run_gpu(enc, rows, frames, tokens, n_classes, ld=None):
    import torch
    from speech_audio_encoder_amd import binding
    dev = torch.from_numpy(rows).cuda()
    if ld is not None and ld != n_classes:
        pad = torch.full((rows.shape[0], ld), float("nan"), dtype=torch.float32, device="cuda")
        pad[:, :n_classes] = dev
        dev = pad
    spans, scores = binding.enc_ctc_align(enc.ctx, dev, frames, tokens, n_classes)
    torch.cuda.synchronize()
    return spans.cpu().numpy(), scores.cpu().numpy()


def build(cases, n_classes):
    rows, frames, tokens = [], [], []
    for i, (t, n, seed, planted) in enumerate(cases):
        lp, tk = workloads.alignment_case(t, n, n_classes, seed, planted=planted)
        rows.append(lp)
        frames.append(t)
        tokens.append(tk)
    rows = np.concatenate(rows) if rows else np.zeros((0, n_classes), np.float32)
    return rows, frames, tokens


def compare(rows, frames, tokens, n_classes, spans, scores, label):
    ref = align.align_batch(rows, frames, tokens, n_classes - 1)
    off = 0
    for b, (sc, sp) in enumerate(ref):
        n = len(tokens[b])
        got_sc = scores[b]
        if np.isneginf(sc):
            assert np.isneginf(got_sc), f"{label} clip {b}: expected no alignment"
            assert (spans[off:off + n] == -1).all()
        else:
            assert got_sc == sc, f"{label} clip {b}: score {got_sc!r} vs {sc!r}"
            np.testing.assert_array_equal(spans[off:off + n], sp, err_msg=f"{label} clip {b}")
        off += n
    say(f"{label}: {len(frames)} clips, {off} tokens, scores and spans exact")


# frames, tokens, seed, planted: tile edges of the state count (S = 2L + 1 at
# 255/257, 511/513, 1023/1025, 2047 states), a clip at the 1,023-token limit,
# no tokens, a single frame, empty clips, too few frames (with and without
# repeats), unplanted noise, and windows longer than the 64-frame backtrack
CASES = [
    (750, 180, 1, True), (200, 60, 2, True), (64, 0, 3, True), (10, 20, 4, True),
    (1, 1, 5, True), (0, 0, 6, True), (300, 127, 7, True), (300, 128, 8, True),
    (700, 255, 9, True), (700, 256, 10, True), (1500, 511, 11, True), (1500, 512, 12, True),
    (2400, 1023, 13, True), (129, 64, 14, False), (65, 65, 15, True), (3, 2, 16, False),
]


def test_align_ragged_exact(enc):
    n_classes = 1000
    rows, frames, tokens = build(CASES, n_classes)
    # a repeat that needs a blank the frames cannot hold
    frames.append(2)
    tokens.append([7, 7])
    rows = np.concatenate([rows, np.zeros((2, n_classes), np.float32)])
    spans, scores = run_gpu(enc, rows, frames, tokens, n_classes)
    compare(rows, frames, tokens, n_classes, spans, scores, "ragged")
    assert np.isneginf(scores[3]) and np.isneginf(scores[-1]) and np.isneginf(scores[5])


def test_align_row_stride_and_full_vocabulary(enc):
    n_classes = oracle.ctc.N_CLASSES
    cases = [(400, 90, 21, True), (180, 40, 22, True), (90, 30, 23, False)]
    rows, frames, tokens = build(cases, n_classes)
    spans, scores = run_gpu(enc, rows, frames, tokens, n_classes, ld=n_classes + 73)
    compare(rows, frames, tokens, n_classes, spans, scores, "full vocabulary, padded rows")


def test_align_batch64_shape(enc):
    # the 64-clip batch's adapter frames (2 P_b per clip), about six tokens a second
    lengths = workloads.batch_lengths(3)
    frames = [2 * oracle.position_count(oracle.frame_count(int(n))) for n in lengths]
    n_classes = 512
    rows, tokens = [], []
    for b, t in enumerate(frames):
        lp, tk = workloads.alignment_case(t, t // 4, n_classes, 1000 + b)
        rows.append(lp)
        tokens.append(tk)
    rows = np.concatenate(rows)
    spans, scores = run_gpu(enc, rows, frames, tokens, n_classes)
    compare(rows, frames, tokens, n_classes, spans, scores, "64-clip batch")


def test_align_repeatable_and_workspace_reuse(enc):
    n_classes = 300
    rows, frames, tokens = build([(500, 100, 31, True), (40, 10, 32, True)], n_classes)
    a = run_gpu(enc, rows, frames, tokens, n_classes)
    small_rows, small_f, small_t = build([(20, 5, 33, True)], n_classes)
    run_gpu(enc, small_rows, small_f, small_t, n_classes)
    b = run_gpu(enc, rows, frames, tokens, n_classes)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_align_errors(enc):
    import torch
    from speech_audio_encoder_amd import binding
    lp = torch.zeros((10, 50), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.EncoderError) as e:
        binding.enc_ctc_align(enc.ctx, lp, [10], [[49]], 50)   # the blank is not a token
    assert e.value.code == binding.ENC_ERR_ARG
    with pytest.raises(binding.EncoderError) as e:
        binding.enc_ctc_align(enc.ctx, lp, [10], [[-1]], 50)
    assert e.value.code == binding.ENC_ERR_ARG
    with pytest.raises(binding.EncoderError) as e:
        binding.enc_ctc_align(enc.ctx, lp, [10], [[1] * 1024], 50)
    assert e.value.code == binding.ENC_ERR_TOO_LONG
    spans, scores = binding.enc_ctc_align(enc.ctx, lp, [], [], 50)   # no clips
    assert spans.numel() == 0 and scores.numel() == 0


def test_align_with_impossible_classes(enc):
    # log-probabilities of -inf (classes that cannot occur in a frame): paths
    # through them are excluded on both sides; a clip whose every path is
    # excluded has no alignment
    n_classes = 64
    rng = np.random.default_rng(41)
    rows, frames, tokens = build([(120, 30, 42, True), (80, 20, 43, False), (50, 10, 44, True)],
                                 n_classes)
    mask = rng.random(rows.shape) < 0.2
    mask[:, n_classes - 1] = False   # the blank stays possible
    rows[mask] = -np.inf
    rows[150:160, :] = -np.inf   # ten frames of the second clip: nothing can be emitted
    spans, scores = run_gpu(enc, rows, frames, tokens, n_classes)
    compare(rows, frames, tokens, n_classes, spans, scores, "impossible classes")
    assert np.isfinite(scores[0]) and np.isneginf(scores[1]) and np.isfinite(scores[2])
