"""Oracle for the Transformer encoder (float32 arithmetic, numpy BLAS).

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Follows "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
section "How audio and speakers reach the language model": the stacked frames
are projected to width 1,280, then 32 Transformer layers with ten attention
heads, QK normalisation, rotary position embeddings and feed-forward
expansion four.  The only norm the page names anywhere is LayerNorm (same
section, speaker branch).

Readings of what the page leaves open (each also listed in the design notes):
  * every linear map has a bias and is stored [out, in] (y = x W^T + b);
  * pre-norm blocks, x + Attn(LN1(x)) then x + FFN(LN2(x)), and a final LN;
  * LayerNorm over the last axis, biased variance, eps = 1e-5, affine;
  * W_qkv rows [0, d) are Q, [d, 2d) K, [2d, 3d) V; head h owns columns
    h*128 .. h*128+127 of each;
  * QK normalisation is a LayerNorm over the 128 dims of each head, one
    (gain, bias) pair for q and one for k shared by all heads, applied before
    the rotation; scores keep the 1/sqrt(128) scale;
  * rotary embedding rotates pairs (i, i+64) by angle p * 10000^(-i/64) for
    position p (0-based within the clip), on q and k only; angles and their
    cosines/sines are formed in float64 and rounded once to float32;
  * bidirectional attention over the clip's whole sequence, no dropout;
  * FFN is two matrices d -> 4d -> d with biases and exact (erf) GELU.

Weights are a dict: ``w_in`` [d, 1024], ``b_in`` [d], ``layers`` (a list of
dicts with ``ln1_g, ln1_b, w_qkv [3d, d], b_qkv, q_g, q_b, k_g, k_b [dh],
w_o [d, d], b_o, ln2_g, ln2_b, w_up [4d, d], b_up, w_down [d, 4d], b_down``),
``lnf_g``, ``lnf_b``.  The head width dh is the length of ``q_g``.
"""

import numpy as np
from scipy.special import erfc

from .frontend import logmel, stack_frames, frame_count, position_count

LN_EPS = 1e-5
ROPE_BASE = 10000.0


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def linear(x, w, b):
    """y = x W^T + b with W stored [out, in]."""
    return _f32(x) @ _f32(w).T + _f32(b)


def layer_norm(x, g, b, eps=LN_EPS):
    """LayerNorm over the last axis: (x - mean) / sqrt(var + eps) * g + b."""
    x = _f32(x)
    mean = x.mean(axis=-1, keepdims=True)
    cen = x - mean
    var = (cen * cen).mean(axis=-1, keepdims=True)
    return (cen / np.sqrt(var + np.float32(eps))) * _f32(g) + _f32(b)


def gelu(x):
    """Exact GELU, x Phi(x) = 0.5 x (1 + erf(x / sqrt 2)).

    Evaluated in float64 as 0.5 x erfc(-x / sqrt 2), the same function written
    without the cancellation of 1 + erf for very negative x.
    """
    x = np.asarray(x, dtype=np.float64)
    return (0.5 * x * erfc(-x / np.sqrt(2.0))).astype(np.float32)


def rope_tables(n_pos, dh):
    """cos, sin [n_pos, dh/2] of p * base^(-i/(dh/2)), built in float64."""
    half = dh // 2
    inv = ROPE_BASE ** (-np.arange(half, dtype=np.float64) / half)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def apply_rope(x, cos, sin):
    """Rotate pairs (i, i + dh/2) of x [T, dh] by the row's angles."""
    x = _f32(x)
    half = x.shape[-1] // 2
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def attention(q, k, v, block=1024):
    """softmax(q k^T / sqrt(dh)) v for one head, exact full-row softmax.

    Query rows are processed ``block`` at a time only to bound memory; each
    row's softmax runs over every key at once.
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    scale = np.float32(1.0 / np.sqrt(q.shape[-1]))
    out = np.empty((q.shape[0], v.shape[-1]), dtype=np.float32)
    for r0 in range(0, q.shape[0], block):
        s = (q[r0:r0 + block] @ k.T) * scale
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        out[r0:r0 + block] = (e @ v) / e.sum(axis=-1, keepdims=True)
    return out


def encoder_layer(x, lw, rows=None):
    """One pre-norm Transformer layer on x [T, d] (float32).

    ``rows`` (optional index array) returns only those output rows; keys and
    values still come from every position, so each returned row equals the
    corresponding row of the full computation.
    """
    x = _f32(x)
    t, d = x.shape
    dh = len(lw["q_g"])
    n_heads = d // dh
    qrows = np.arange(t) if rows is None else np.asarray(rows)
    a = layer_norm(x, lw["ln1_g"], lw["ln1_b"])
    w_qkv, b_qkv = _f32(lw["w_qkv"]), _f32(lw["b_qkv"])
    kv = linear(a, w_qkv[d:], b_qkv[d:])
    qx = linear(a[qrows], w_qkv[:d], b_qkv[:d])
    cos, sin = rope_tables(t, dh)
    heads = []
    for h in range(n_heads):
        q = qx[:, h * dh:(h + 1) * dh]
        k = kv[:, h * dh:(h + 1) * dh]
        v = kv[:, d + h * dh:d + (h + 1) * dh]
        q = apply_rope(layer_norm(q, lw["q_g"], lw["q_b"]), cos[qrows], sin[qrows])
        k = apply_rope(layer_norm(k, lw["k_g"], lw["k_b"]), cos, sin)
        heads.append(attention(q, k, v))
    o = np.concatenate(heads, axis=-1)
    xr = x[qrows] + linear(o, lw["w_o"], lw["b_o"])
    a = layer_norm(xr, lw["ln2_g"], lw["ln2_b"])
    u = gelu(linear(a, lw["w_up"], lw["b_up"]))
    return xr + linear(u, lw["w_down"], lw["b_down"])


def encode_from_logmel(feats, weights, n_layers=None, rows=None):
    """Stack, project and run the encoder on one clip's log-mel [F, 128].

    ``rows`` limits the output (and the last layer's queries) to those
    positions; earlier layers always run on every position.
    """
    layers = weights["layers"] if n_layers is None else weights["layers"][:n_layers]
    s = stack_frames(feats)
    d = weights["w_in"].shape[0]
    if s.shape[0] == 0:
        return np.zeros((0, d), dtype=np.float32)
    x = linear(s, weights["w_in"], weights["b_in"])
    if rows is not None and not layers:
        x = x[np.asarray(rows)]
    for i, lw in enumerate(layers):
        last = i == len(layers) - 1
        x = encoder_layer(x, lw, rows if last else None)
    return layer_norm(x, weights["lnf_g"], weights["lnf_b"])


def encode(x, weights, n_layers=None, rows=None):
    """Embeddings [ceil(F/8), d] of one clip's waveform x (or only ``rows``)."""
    return encode_from_logmel(logmel(x), weights, n_layers, rows)


def encode_windows(x, weights, core, context, n_layers=None):
    """Embeddings [P, d] of one clip encoded in local attention windows.

    The encoder is trained on 30-second chunks and served with local windows
    of 500 positions plus 50 of context on either side ("Nemotron 3.5
    Transcribe: From Recorded Speech to Dataset Audits", section "Local
    encoder windows, recording-wide language context").  Position p belongs
    to window w = p // core; the window's sequence is positions
    [max(0, w core - context), min(P, (w + 1) core + context)) of the clip's
    stacked features, encoded on its own (attention inside it, rotary
    positions from its first position); p takes the row computed in its own
    window.  context = 0 gives non-overlapping chunks.
    """
    feats = logmel(x)
    n_frames = feats.shape[0]
    P = position_count(n_frames)
    d = weights["w_in"].shape[0]
    out = np.zeros((P, d), dtype=np.float32)
    for c0 in range(0, P, core):
        st = max(0, c0 - context)
        en = min(P, c0 + core + context)
        # positions st .. en-1 stack frames 8 st .. 8 en - 1 (zeros past the clip)
        y = encode_from_logmel(feats[8 * st:min(n_frames, 8 * en)], weights, n_layers)
        c1 = min(P, c0 + core)
        out[c0:c1] = y[c0 - st:c1 - st]
    return out


def encode_batch(audio, lengths, weights, n_layers=None):
    """[B, P(max length), d] embeddings; each clip encoded alone, rows >= P_b zero."""
    lengths = [int(n) for n in lengths]
    d = weights["w_in"].shape[0]
    pmax = position_count(frame_count(max(lengths))) if lengths else 0
    out = np.zeros((len(lengths), pmax, d), dtype=np.float32)
    for b, n in enumerate(lengths):
        e = encode(np.asarray(audio[b, :n]), weights, n_layers)
        out[b, :e.shape[0]] = e
    return out


def parameter_count(d=1280, n_layers=32, dh=128, ffn_mult=4, in_dim=1024,
                    gated_ffn=False):
    """Parameter count of this reading of the encoder (input projection,
    layers, final norm).  ``gated_ffn`` counts the three-matrix alternative."""
    f = ffn_mult * d
    per_layer = (2 * d                      # LN1
                 + 3 * d * d + 3 * d        # QKV
                 + 4 * dh                   # QK norms
                 + d * d + d                # output projection
                 + 2 * d                    # LN2
                 + (3 * d * f + 2 * f + d if gated_ffn else 2 * d * f + f + d))  # FFN
    return in_dim * d + d + n_layers * per_layer + 2 * d
