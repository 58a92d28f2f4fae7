"""Oracle for speaker-activity fusion and the identity connector.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Follows "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
section "How audio and speakers reach the language model": speaker activity
for up to eight slots is aligned to the ASR grid, thresholded at 0.5 and
passed through a learned LayerNorm over the speaker dimension; a fixed
sinusoidal speaker kernel (saved scale 1) maps the eight slot values to the
acoustic width, and the result is added to the ASR states, keeping the number
of positions and the width 1,280.  One learned linear projection (the
identity connector, no temporal downsampling) then maps the fused states to
the language model's width, 2,688 (the width the section "What the 52
backbone blocks actually do" gives for the backbone's projections).

The fusion and connector formulas did not survive the page's extraction;
this oracle takes the plainest reading of the prose (listed in the design
notes as well):
  * activity arrives on the ASR grid already (one 8-vector of probabilities
    per 80 ms position), so "pools/aligns" is the identity here;
  * thresholding gives indicators 1 where the probability is > 0.5, else 0;
  * LayerNorm over the 8 slots as for every other norm: biased variance,
    eps = 1e-5, learned gain and bias of length 8;
  * the sinusoidal kernel is the sinusoid table of the original Transformer
    (Vaswani et al. 2017, section 3.5) with the slot index s = 0..7 in place
    of the position: K[s, 2i] = sin(s w_i), K[s, 2i+1] = cos(s w_i),
    w_i = 10000^(-2i/1280), times the saved scale;
  * fused = H + LN(indicators) K (a [8] x [8, 1280] product per position);
  * connector: z = fused W_c^T + b_c with W_c [2688, 1280].
Arithmetic: the kernel table in float64, everything else float32 (the
encoder oracle's precision).
"""

import numpy as np

from .encoder import encode, encode_windows, layer_norm, linear

N_SPEAKERS = 8
SPEAKER_BASE = 10000.0
THRESHOLD = 0.5


def speaker_kernel(d=1280, n_slots=N_SPEAKERS, scale=1.0):
    """[n_slots, d] table: slot s, column 2i -> sin(s w_i), 2i+1 -> cos(s w_i)."""
    s = np.arange(n_slots, dtype=np.float64)[:, None]
    w = SPEAKER_BASE ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    k = np.empty((n_slots, d), dtype=np.float64)
    k[:, 0::2] = np.sin(s * w)
    k[:, 1::2] = np.cos(s * w)
    return k * scale


def speaker_indicators(activity):
    """Activity probabilities [..., 8] -> 0/1 indicators (> 0.5), float32."""
    return (np.asarray(activity, dtype=np.float32) > np.float32(THRESHOLD)).astype(np.float32)


def speaker_features(activity, ln_g, ln_b):
    """LayerNorm over the speaker slots of the thresholded activity [T, 8]."""
    return layer_norm(speaker_indicators(activity), ln_g, ln_b)


def fuse_speakers(h, activity, cw):
    """ASR states h [T, d] plus the speaker term of activity [T, 8]."""
    h = np.asarray(h, dtype=np.float32)
    n = speaker_features(activity, cw["spk_ln_g"], cw["spk_ln_b"])
    k = speaker_kernel(h.shape[1], scale=cw.get("speaker_scale", 1.0)).astype(np.float32)
    return h + n @ k


def connector(fused, cw):
    """Linear map to the language model's width."""
    return linear(fused, cw["w_conn"], cw["b_conn"])


def encode_fused(x, weights, activity, cw, n_layers=None, windows=None):
    """Waveform of one clip -> language-model input rows [P, out_dim].
    activity: [P, 8] on the ASR grid.  windows: None (whole clip) or
    (core, context) as in encode_windows."""
    if windows is None:
        h = encode(x, weights, n_layers=n_layers)
    else:
        h = encode_windows(x, weights, windows[0], windows[1], n_layers=n_layers)
    assert activity.shape == (h.shape[0], N_SPEAKERS)
    return connector(fuse_speakers(h, activity, cw), cw)
