"""Pins of the CTC forced-alignment oracle (oracle/align.py).

"Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
"4. Use alignment and audio questions as supporting evidence" (forced
alignment of the generated word sequence onto the CTC frame probabilities).
The oracle is pinned by brute force over every valid path on small cases, by
planted paths with known answers, and against torch's CTC loss (the sum over
the same set of paths): the best path can never beat the total, reaches it
when one path holds all the probability, and both agree on which sequences
cannot be aligned.
"""

import itertools

import numpy as np
import pytest
import torch

from oracle import align

BLANK = 5   # classes 0..5, blank last


def valid_path(states, s_count, skip):
    if states[0] not in (0, 1) or states[-1] not in (s_count - 1, s_count - 2):
        return False
    for a, b in zip(states, states[1:]):
        if b == a or b == a + 1:
            continue
        if b == a + 2 and skip[b]:
            continue
        return False
    return True


def brute_force(lp, tokens, blank):
    """Best score and state path over every valid path, scores summed in frame
    order in float32 (ties: the first path in lexicographic order)."""
    lab = align.extended_labels(tokens, blank)
    skip = align.skip_allowed(tokens)
    s_count = len(lab)
    best, arg = None, None
    for states in itertools.product(range(s_count), repeat=lp.shape[0]):
        if not valid_path(states, s_count, skip):
            continue
        sc = np.float32(0.0)
        for t, s in enumerate(states):
            sc = np.float32(sc + lp[t, lab[s]])
        if best is None or sc > best:
            best, arg = sc, states
    return best, arg


@pytest.mark.parametrize("seed,t_count,tokens", [
    (0, 4, [1, 2]), (1, 5, [1, 1]), (2, 6, [3, 1, 3]), (3, 5, [0]), (4, 6, [2, 2, 4]),
    (5, 3, [4, 0, 1]), (6, 7, [0, 1]), (7, 2, [])])
def test_brute_force_small(seed, t_count, tokens):
    rng = np.random.default_rng(seed)
    lp = rng.normal(-3.0, 2.0, size=(t_count, BLANK + 1)).astype(np.float32)
    score, states, spans = align.ctc_forced_align(lp, tokens, BLANK)
    bf, path = brute_force(lp, tokens, BLANK)
    assert bf is not None
    assert score == bf
    assert list(states) == list(path)
    for i in range(len(tokens)):
        frames = [t for t, s in enumerate(states) if s == 2 * i + 1]
        assert spans[i].tolist() == [frames[0], frames[-1]]


def planted_lp(classes, n_classes=BLANK + 1, low=-50.0):
    lp = np.full((len(classes), n_classes), low, dtype=np.float32)
    lp[np.arange(len(classes)), classes] = 0.0
    return lp


def test_planted_path_recovered():
    # frames: blank, 1, 1, blank, 2, 2, 2, blank, 2 (a repeat after a blank)
    classes = [BLANK, 1, 1, BLANK, 2, 2, 2, BLANK, 2]
    score, states, spans = align.ctc_forced_align(planted_lp(classes), [1, 2, 2], BLANK)
    assert score == 0.0
    assert states.tolist() == [0, 1, 1, 2, 3, 3, 3, 4, 5]
    assert spans.tolist() == [[1, 2], [4, 6], [8, 8]]


def test_repeats_need_a_blank():
    lp = planted_lp([3, 3])
    score, states, spans = align.ctc_forced_align(lp, [3, 3], BLANK)
    assert score == -np.inf and (spans == -1).all() and (states == -1).all()
    assert align.min_frames([3, 3]) == 3 and align.min_frames([3, 4, 4, 4]) == 6
    score, states, spans = align.ctc_forced_align(planted_lp([3, BLANK, 3]), [3, 3], BLANK)
    assert score == 0.0 and states.tolist() == [1, 2, 3] and spans.tolist() == [[0, 0], [2, 2]]


def test_empty_sequence_is_all_blank():
    rng = np.random.default_rng(9)
    lp = rng.normal(-2.0, 1.0, size=(7, BLANK + 1)).astype(np.float32)
    score, states, spans = align.ctc_forced_align(lp, [], BLANK)
    total = np.float32(0.0)
    for t in range(7):
        total = np.float32(total + lp[t, BLANK])
    assert score == total and (states == 0).all() and spans.shape == (0, 2)


def test_all_zero_scores_give_a_valid_path():
    lp = np.zeros((9, BLANK + 1), dtype=np.float32)
    tokens = [1, 2, 2, 0]
    score, states, spans = align.ctc_forced_align(lp, tokens, BLANK)
    assert score == 0.0
    assert valid_path(list(states), 2 * len(tokens) + 1, align.skip_allowed(tokens))
    assert (spans[:, 0] <= spans[:, 1]).all() and (np.diff(spans[:, 0]) > 0).all()


def torch_ctc_logprob(lp, tokens, blank):
    """log of the total probability of all paths spelling tokens (torch)."""
    t = torch.from_numpy(lp.astype(np.float64)).unsqueeze(1)   # [T, 1, C]
    tg = torch.tensor([tokens], dtype=torch.long)
    loss = torch.nn.functional.ctc_loss(t, tg, torch.tensor([lp.shape[0]]),
                                        torch.tensor([len(tokens)]), blank=blank,
                                        reduction="sum", zero_infinity=False)
    return -float(loss)


@pytest.mark.parametrize("seed", range(6))
def test_best_path_bounded_by_torch_total(seed):
    rng = np.random.default_rng(100 + seed)
    t_count = int(rng.integers(6, 30))
    n_tok = int(rng.integers(1, max(2, t_count // 3)))
    tokens = [int(v) for v in rng.integers(0, 3, size=n_tok)]   # many repeats
    z = rng.normal(0.0, 2.0, size=(t_count, BLANK + 1))
    lp = (z - np.log(np.exp(z).sum(axis=1, keepdims=True))).astype(np.float32)
    score, _, _ = align.ctc_forced_align(lp, tokens, BLANK)
    total = torch_ctc_logprob(lp, tokens, BLANK)
    if t_count < align.min_frames(tokens):
        assert score == -np.inf and total == -np.inf
    else:
        assert np.isfinite(score) and score <= total + 1e-4


def test_single_dominant_path_matches_torch_total():
    # one path holds (almost) all the probability: its score equals the total
    classes = [BLANK, 0, 0, 1, BLANK, 1, 2, 2, BLANK]
    lp = planted_lp(classes, low=-40.0)
    lp = lp - np.log(np.exp(lp.astype(np.float64)).sum(axis=1, keepdims=True)).astype(np.float32)
    tokens = [0, 1, 1, 2]
    score, states, spans = align.ctc_forced_align(lp, tokens, BLANK)
    assert spans.tolist() == [[1, 2], [3, 3], [5, 5], [6, 7]]
    assert abs(score - torch_ctc_logprob(lp, tokens, BLANK)) < 1e-3


def test_infeasible_agrees_with_torch():
    lp = planted_lp([2, 2, 2])
    lp = lp - np.log(np.exp(lp.astype(np.float64)).sum(axis=1, keepdims=True)).astype(np.float32)
    for tokens in ([2, 2, 2], [0, 1, 2, 3]):
        score, _, _ = align.ctc_forced_align(lp, tokens, BLANK)
        assert score == -np.inf and torch_ctc_logprob(lp, tokens, BLANK) == -np.inf


def test_align_batch_splits_rows():
    rng = np.random.default_rng(3)
    frames = [5, 0, 7]
    toks = [[1, 2], [], [0, 0, 3]]
    rows = rng.normal(-2.0, 1.0, size=(sum(frames), BLANK + 1)).astype(np.float32)
    got = align.align_batch(rows, frames, toks, BLANK)
    assert got[1][0] == -np.inf
    s0, _, sp0 = align.ctc_forced_align(rows[:5], toks[0], BLANK)
    s2, _, sp2 = align.ctc_forced_align(rows[5:], toks[2], BLANK)
    assert got[0][0] == s0 and (got[0][1] == sp0).all()
    assert got[2][0] == s2 and (got[2][1] == sp2).all()
