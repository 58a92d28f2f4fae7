"""Oracle for CTC forced alignment of a given token sequence.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

"Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
"4. Use alignment and audio questions as supporting evidence": after
decoding, a forced alignment maps the supplied generated word sequence onto
the CTC adapter's frame probabilities (40 ms grid), which yields the word
timestamps; the same section notes that such a dynamic program can force
wrong words onto plausible frames, and that a failed alignment is a review
signal.

Readings of what the page leaves open (also in the design notes):
  * the alignment is the single most probable CTC path that spells the
    token sequence (Viterbi, max-product), over the standard CTC topology:
    the extended sequence blank, y1, blank, y2, ..., yL, blank (S = 2L + 1
    states); a path starts in state 0 or 1, ends in state S - 1 or S - 2,
    and from state s moves to s, s + 1, or s + 2 when state s + 2 is a token
    different from the token in state s (a blank must separate repeats);
  * path score: the sum over frames of the log-probability of the path's
    class in that frame, accumulated frame by frame in float32 (the score of
    frame t's best path into state s is lp[t, class(s)] + the best of its
    predecessors' scores); ties between predecessors go to the state that
    stays, then to s - 1, then to s - 2, and between the two final states to
    the blank;
  * output per token: the first and the last frame the path spends in that
    token's state (a token always gets at least one frame); grouping tokens
    into words is the caller's;
  * a sequence that cannot fit (fewer frames than tokens plus repeated
    neighbours) has no alignment: score -inf, spans (-1, -1).
The decisions are taken in float32, as the adapter's log-probabilities are.
"""

import numpy as np

NEG_INF = np.float32(-np.inf)


def extended_labels(tokens, blank):
    """Class of each state of the extended sequence (blank, y1, ..., yL, blank)."""
    tokens = [int(t) for t in tokens]
    lab = np.full(2 * len(tokens) + 1, blank, dtype=np.int64)
    lab[1::2] = tokens
    return lab


def skip_allowed(tokens):
    """State s may be entered from s - 2: s is a token state whose token
    differs from the previous token (so no blank is skipped between repeats)."""
    tokens = [int(t) for t in tokens]
    s_count = 2 * len(tokens) + 1
    ok = np.zeros(s_count, dtype=bool)
    for i in range(1, len(tokens)):
        ok[2 * i + 1] = tokens[i] != tokens[i - 1]
    return ok


def min_frames(tokens):
    """Fewest frames a path spelling `tokens` needs: one per token plus one
    blank between equal neighbours."""
    tokens = [int(t) for t in tokens]
    return len(tokens) + sum(1 for a, b in zip(tokens, tokens[1:]) if a == b)


def ctc_forced_align(lp, tokens, blank):
    """Viterbi alignment of `tokens` to log-probabilities lp [T, V].

    Returns (score, states, spans): the best path's float32 score, its state
    per frame (int array [T], -1 when infeasible) and, per token, the first
    and last frame of its state (int array [L, 2], -1 when infeasible)."""
    lp = np.asarray(lp, dtype=np.float32)
    t_count = lp.shape[0]
    tokens = [int(t) for t in tokens]
    n_tok = len(tokens)
    spans = np.full((n_tok, 2), -1, dtype=np.int64)
    if t_count < max(1, min_frames(tokens)):
        return NEG_INF, np.full(t_count, -1, dtype=np.int64), spans
    lab = extended_labels(tokens, blank)
    skip = skip_allowed(tokens)
    s_count = len(lab)
    delta = np.full(s_count, NEG_INF, dtype=np.float32)
    delta[0] = lp[0, lab[0]]
    if s_count > 1:
        delta[1] = lp[0, lab[1]]
    back = np.zeros((t_count, s_count), dtype=np.int8)   # 0 stay, 1 from s-1, 2 from s-2
    for t in range(1, t_count):
        stay = delta
        m1 = np.full(s_count, NEG_INF, dtype=np.float32)
        m1[1:] = delta[:-1]
        m2 = np.full(s_count, NEG_INF, dtype=np.float32)
        m2[2:] = delta[:-2]
        m2 = np.where(skip, m2, NEG_INF).astype(np.float32)
        best = stay.copy()
        bp = np.zeros(s_count, dtype=np.int8)
        take1 = m1 > best
        best = np.where(take1, m1, best)
        bp = np.where(take1, np.int8(1), bp)
        take2 = m2 > best
        best = np.where(take2, m2, best)
        bp = np.where(take2, np.int8(2), bp)
        back[t] = bp
        delta = (lp[t, lab] + best).astype(np.float32)
    # end in the final blank or the last token; ties to the blank
    s = s_count - 1
    if s_count > 1 and delta[s_count - 2] > delta[s_count - 1]:
        s = s_count - 2
    score = delta[s]
    if not np.isfinite(score):
        return NEG_INF, np.full(t_count, -1, dtype=np.int64), spans
    states = np.empty(t_count, dtype=np.int64)
    for t in range(t_count - 1, -1, -1):
        states[t] = s
        s -= int(back[t, s])
    for t, st in enumerate(states):
        if st % 2 == 1:
            i = st // 2
            if spans[i, 0] < 0:
                spans[i, 0] = t
            spans[i, 1] = t
    return np.float32(score), states, spans


def align_batch(lp_rows, frames, tokens_per_clip, blank):
    """Clip-packed rows (clip b's T_b frames after the clips before it) ->
    per clip (score, spans), as ctc_forced_align."""
    out = []
    r = 0
    for t_count, toks in zip(frames, tokens_per_clip):
        score, _, spans = ctc_forced_align(lp_rows[r:r + t_count], toks, blank)
        out.append((score, spans))
        r += t_count
    return out
