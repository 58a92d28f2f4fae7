"""Oracle for the CTC timestamp adapter's forward pass.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

"Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits", section
"4. Use alignment and audio questions as supporting evidence": an adapter of
roughly 50M parameters reads the unfused ASR states (width 1,280, 80 ms
grid); a stride-two transposed convolution upsamples them to a 40 ms grid;
two Transformer layers with 16 heads follow, then a projection to a
23,862-token vocabulary plus the CTC blank, whose frame probabilities a
forced alignment consumes.

Readings of what the page leaves open (also in the design notes):
  * input: the encoder's output (final LayerNorm included), before speaker
    fusion -- the "unfused" states;
  * upsampling: ConvTranspose1d(1280 -> 1280, kernel 2, stride 2, bias), so
    output frame 2t + j = H[t] W_j + b (j = 0, 1; the taps do not overlap);
  * the two layers are the encoder's block type (pre-norm, QKV with biases,
    QK-norm over each head's 80 dims, rotary embedding of pairs (i, i + 40)
    at the frame's position on the 40 ms grid, bidirectional attention over
    the clip, output projection, GELU FFN) with 16 heads of width 80 and a
    feed-forward width of 1,280 (expansion 1: with it the adapter has 53.5M
    parameters, the stated "approximately 50M"; expansion 4 would give 73M);
  * a final LayerNorm, then the projection to 23,863 classes (blank last) and
    log-softmax over the classes.
Arithmetic float32 (the encoder oracle's), log-softmax in float64.
"""

import numpy as np

from .encoder import encode, encode_windows, encoder_layer, layer_norm, linear

N_CLASSES = 23_863   # 23,862 tokens + blank


def upsample(h, w_conv, b_conv):
    """Stride-2, kernel-2 transposed convolution: [T, d] -> [2T, d].
    w_conv [2, d_out, d_in] (tap j maps H[t] to output frame 2t + j)."""
    h = np.asarray(h, dtype=np.float32)
    t, _ = h.shape
    d_out = w_conv.shape[1]
    out = np.empty((2 * t, d_out), dtype=np.float32)
    for j in range(2):
        out[j::2] = linear(h, w_conv[j], b_conv)
    return out


def log_softmax(z):
    z = np.asarray(z, dtype=np.float64)
    m = z.max(axis=-1, keepdims=True)
    return (z - m - np.log(np.exp(z - m).sum(axis=-1, keepdims=True))).astype(np.float32)


def adapter_from_states(h, cw):
    """Adapter on encoder states h [P, 1280] -> log-probabilities [2P, 23863]."""
    x = upsample(h, cw["w_conv"], cw["b_conv"])
    for lw in cw["layers"]:
        x = encoder_layer(x, lw)
    x = layer_norm(x, cw["lnf_g"], cw["lnf_b"])
    return log_softmax(linear(x, cw["w_out"], cw["b_out"]))


def ctc_logprobs(x, weights, cw, windows=None):
    """Waveform of one clip -> CTC log-probabilities on the 40 ms grid."""
    if windows is None:
        h = encode(x, weights)
    else:
        h = encode_windows(x, weights, windows[0], windows[1])
    if h.shape[0] == 0:
        return np.zeros((0, cw["w_out"].shape[0]), dtype=np.float32)
    return adapter_from_states(h, cw)


def parameter_count(d=1280, heads=16, ffn=1280, n_layers=2, n_classes=N_CLASSES):
    dh = d // heads
    conv = 2 * d * d + d
    layer = (2 * d) + (3 * d * d + 3 * d) + 4 * dh + (d * d + d) + (2 * d) \
        + (ffn * d + ffn) + (d * ffn + d)
    return conv + n_layers * layer + 2 * d + n_classes * d + n_classes
