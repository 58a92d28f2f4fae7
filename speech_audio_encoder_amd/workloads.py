"""Seeded synthetic inputs: waveforms, clip lengths and random-init weights.

This module only draws inputs.  It holds none of the encoder's arithmetic
(no framing, transform, mel, norm or attention) and imports neither the HIP
library nor the oracle, so both sides of a parity test can take their inputs
from it.

Workloads (all 16 kHz mono float32, weights N(0, 0.02^2), biases 0, gains 1):
  * ``tiny``    1 x 1.0 s sinusoid mixture, 2 layers, float32 weights;
  * ``clip30``  1 x 30 s sinusoid mixture, 32 layers, weights stored in bf16;
  * ``batch64`` 64 clips of U{5 s .. 30 s} (80,000..480,000 samples), padded
                to the longest; 32 layers, bf16 weights;
  * ``long10m`` 1 x 600 s segment mixture, 32 layers, bf16 weights;
  * ``hour``    1 x 3,600 s segment mixture, 32 layers, bf16 weights.

Sinusoid mixture: three tones with frequencies U(100, 4000) Hz, amplitudes
U(0.1, 0.3) and phases U(0, 2 pi), plus Gaussian noise of sigma 0.01.
Segment mixture: segments of U(2, 8) s (whole samples) cycling tone mixture
-> amplitude-modulated noise 0.1 (0.5 + 0.5 sin(2 pi f_m t + phi)) eps with
f_m ~ U(2, 8) Hz -> silence 1e-4 eps -> tone mixture ...; the last segment is
cut to the exact length.

Weights are drawn tensor by tensor from ``numpy.random.default_rng`` seeded
with (1234, layer + 1, tensor id), so a prefix of layers is the same draw whatever
the total depth.  "Stored in bf16" means each drawn value is rounded to the
nearest bfloat16 (ties to even) and kept as a float32 holding that value.
"""

import numpy as np

SAMPLE_RATE = 16000
D_MODEL = 1280
N_HEADS = 10
HEAD_DIM = 128
FFN_DIM = 4 * D_MODEL
IN_DIM = 1024
WEIGHT_SEED = 1234
WEIGHT_STD = 0.02

WORKLOADS = {
    # name: (audio seed, kind, n_layers, bf16 weights)
    "tiny": (1, "tone", 2, False),
    "clip30": (2, "tone", 32, True),
    "batch64": (3, "tone_batch", 32, True),
    "long10m": (4, "segments", 32, True),
    "hour": (5, "segments", 32, True),
}
WORKLOAD_ORDER = ["tiny", "clip30", "batch64", "long10m", "hour"]

_DURATION_S = {"tiny": 1.0, "clip30": 30.0, "long10m": 600.0, "hour": 3600.0}

# (name, shape kind, layer-local id); order is fixed and never reused.
_LAYER_TENSORS = [
    ("ln1_g", "gain", 0), ("ln1_b", "bias_d", 1),
    ("w_qkv", "w_qkv", 2), ("b_qkv", "bias_qkv", 3),
    ("q_g", "gain_h", 4), ("q_b", "bias_h", 5),
    ("k_g", "gain_h", 6), ("k_b", "bias_h", 7),
    ("w_o", "w_o", 8), ("b_o", "bias_d", 9),
    ("ln2_g", "gain", 10), ("ln2_b", "bias_d", 11),
    ("w_up", "w_up", 12), ("b_up", "bias_f", 13),
    ("w_down", "w_down", 14), ("b_down", "bias_d", 15),
]


def tone_mixture(rng, n):
    """Three random tones plus N(0, 0.01^2) noise, n samples, float32."""
    t = np.arange(n, dtype=np.float64) / SAMPLE_RATE
    freqs = rng.uniform(100.0, 4000.0, size=3)
    amps = rng.uniform(0.1, 0.3, size=3)
    phases = rng.uniform(0.0, 2.0 * np.pi, size=3)
    x = np.zeros(n, dtype=np.float64)
    for f, a, p in zip(freqs, amps, phases):
        x += a * np.sin(2.0 * np.pi * f * t + p)
    x += 0.01 * rng.standard_normal(n)
    return x.astype(np.float32)


def _am_noise(rng, n):
    t = np.arange(n, dtype=np.float64) / SAMPLE_RATE
    fm = rng.uniform(2.0, 8.0)
    ph = rng.uniform(0.0, 2.0 * np.pi)
    env = 0.5 + 0.5 * np.sin(2.0 * np.pi * fm * t + ph)
    return (0.1 * env * rng.standard_normal(n)).astype(np.float32)


def _silence(rng, n):
    return (1e-4 * rng.standard_normal(n)).astype(np.float32)


def segment_mixture(rng, n):
    """Cycling 2-8 s segments: tones, AM noise, near-silence; n samples."""
    out = np.empty(n, dtype=np.float32)
    makers = (tone_mixture, _am_noise, _silence)
    pos, kind = 0, 0
    while pos < n:
        seg = int(rng.integers(2 * SAMPLE_RATE, 8 * SAMPLE_RATE + 1))
        seg = min(seg, n - pos)
        out[pos:pos + seg] = makers[kind](rng, seg)
        pos += seg
        kind = (kind + 1) % 3
    return out


def batch_lengths(seed=3, batch=64):
    """Clip lengths for the 64-clip batch: uniform integers in [80,000, 480,000]."""
    rng = np.random.default_rng(seed)
    return rng.integers(80_000, 480_000 + 1, size=batch).astype(np.int64)


def workload_audio(name):
    """(audio [B, N_max] float32 zero-padded, lengths int64 [B]) for a workload."""
    seed, kind, _, _ = WORKLOADS[name]
    if kind == "tone_batch":
        lengths = batch_lengths(seed)
        audio = np.zeros((len(lengths), int(lengths.max())), dtype=np.float32)
        for b, n in enumerate(lengths):
            audio[b, :n] = tone_mixture(np.random.default_rng((seed, b)), int(n))
        return audio, lengths
    n = int(round(_DURATION_S[name] * SAMPLE_RATE))
    rng = np.random.default_rng(seed)
    x = tone_mixture(rng, n) if kind == "tone" else segment_mixture(rng, n)
    return x[None, :], np.array([n], dtype=np.int64)


def custom_audio(lengths, seed, kind="tone"):
    """Padded batch of tone (or segment) mixtures with the given lengths."""
    lengths = np.asarray(lengths, dtype=np.int64)
    nmax = int(lengths.max()) if len(lengths) else 0
    audio = np.zeros((len(lengths), nmax), dtype=np.float32)
    maker = tone_mixture if kind == "tone" else segment_mixture
    for b, n in enumerate(lengths):
        if n > 0:
            audio[b, :n] = maker(np.random.default_rng((seed, b)), int(n))
    return audio, lengths


def round_bf16(a, inplace=False):
    """Nearest bfloat16 value (ties to even) of float32 a, kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not inplace:
        a = a.copy()
    if not np.all(np.isfinite(a)):
        raise ValueError("round_bf16 expects finite values")
    u = a.view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    u += lsb
    u += np.uint32(0x7FFF)
    u &= np.uint32(0xFFFF0000)
    return a


def _shape(kind, d, dh, f, in_dim):
    return {
        "gain": (d,), "bias_d": (d,), "gain_h": (dh,), "bias_h": (dh,),
        "w_qkv": (3 * d, d), "bias_qkv": (3 * d,), "w_o": (d, d),
        "w_up": (f, d), "bias_f": (f,), "w_down": (d, f), "w_in": (d, in_dim),
    }[kind]


def _draw(kind, shape, rng, perturb):
    if kind.startswith("w_"):
        out = np.empty(shape, dtype=np.float32)
        rng.standard_normal(out=out, dtype=np.float32)
        out *= np.float32(WEIGHT_STD)
        return out
    if kind.startswith("gain"):
        if perturb:
            return (1.0 + 0.1 * rng.standard_normal(shape)).astype(np.float32)
        return np.ones(shape, dtype=np.float32)
    if perturb:
        return (0.1 * rng.standard_normal(shape)).astype(np.float32)
    return np.zeros(shape, dtype=np.float32)


def make_weights(n_layers, bf16=True, perturb=False, d=D_MODEL, dh=HEAD_DIM,
                 ffn=FFN_DIM, in_dim=IN_DIM, seed=WEIGHT_SEED):
    """Random-init weights as a dict (see the oracle's encoder for the keys).

    ``perturb`` replaces the zero biases and unit gains by N(0, 0.1^2) and
    1 + N(0, 0.1^2) draws, so that every bias and affine term is exercised.
    """
    def tensor(layer, tid, kind):
        # layer -1 holds the tensors outside the stack; SeedSequence needs >= 0
        key = (seed, layer + 1, tid)
        if perturb and not kind.startswith("w_"):
            key = key + (1,)
        rng = np.random.default_rng(key)
        a = _draw(kind, _shape(kind, d, dh, ffn, in_dim), rng, perturb)
        return round_bf16(a, inplace=True) if bf16 else a

    w = {
        "w_in": tensor(-1, 0, "w_in"),
        "b_in": tensor(-1, 1, "bias_d"),
        "lnf_g": tensor(-1, 2, "gain"),
        "lnf_b": tensor(-1, 3, "bias_d"),
        "layers": [],
    }
    for layer in range(n_layers):
        w["layers"].append({name: tensor(layer, tid, kind)
                            for name, kind, tid in _LAYER_TENSORS})
    return w


def workload_weights(name, n_layers=None, perturb=False):
    """Weights for a workload (optionally only its first n_layers layers)."""
    _, _, depth, bf16 = WORKLOADS[name]
    return make_weights(depth if n_layers is None else n_layers, bf16=bf16,
                        perturb=perturb)


# ------------------------------------------------- speaker activity, connector
N_SPEAKERS = 8
LLM_DIM = 2688


def speaker_activity(n_positions, seed, max_speakers=4):
    """Synthetic speaker-activity probabilities [n_positions, 8] float32 on the
    80 ms grid: a conversation of 1-4 speakers in turns of 1-8 s (12-100
    positions), with occasional overlap of a second speaker; active slots
    draw probabilities U(0.6, 1.0), inactive ones U(0.0, 0.4), and a few
    positions sit near the 0.5 threshold (U(0.45, 0.55))."""
    rng = np.random.default_rng((seed, 9))
    act = rng.uniform(0.0, 0.4, (n_positions, N_SPEAKERS)).astype(np.float32)
    n_spk = int(rng.integers(1, max_speakers + 1))
    slots = rng.choice(N_SPEAKERS, n_spk, replace=False)
    p = 0
    while p < n_positions:
        turn = int(rng.integers(12, 101))
        who = int(rng.choice(slots))
        end = min(n_positions, p + turn)
        act[p:end, who] = rng.uniform(0.6, 1.0, end - p)
        if n_spk > 1 and rng.uniform() < 0.3:
            other = int(rng.choice([s for s in slots if s != who]))
            o0 = int(rng.integers(p, end))
            act[o0:end, other] = rng.uniform(0.6, 1.0, end - o0)
        p = end
    near = rng.uniform(size=n_positions) < 0.02
    act[near] = rng.uniform(0.45, 0.55, (int(near.sum()), N_SPEAKERS))
    return act


def make_connector_weights(bf16=True, perturb=False, d=D_MODEL, out_dim=LLM_DIM,
                           seed=WEIGHT_SEED):
    """Random-init speaker LayerNorm (gain 1, bias 0; N(1, 0.1^2) and
    N(0, 0.1^2) draws with perturb) and connector (N(0, 0.02^2) weights,
    zero or N(0, 0.1^2) bias), speaker-kernel scale 1."""
    def rng(tid):
        return np.random.default_rng((seed, 1000, tid))
    g = np.ones(N_SPEAKERS, np.float32)
    b = np.zeros(N_SPEAKERS, np.float32)
    bc = np.zeros(out_dim, np.float32)
    if perturb:
        g = (1.0 + 0.1 * rng(0).standard_normal(N_SPEAKERS)).astype(np.float32)
        b = (0.1 * rng(1).standard_normal(N_SPEAKERS)).astype(np.float32)
        bc = (0.1 * rng(3).standard_normal(out_dim)).astype(np.float32)
    w = (WEIGHT_STD * rng(2).standard_normal((out_dim, d))).astype(np.float32)
    cw = {"spk_ln_g": g, "spk_ln_b": b, "w_conn": w, "b_conn": bc, "speaker_scale": 1.0}
    if bf16:
        for k in ("spk_ln_g", "spk_ln_b", "w_conn", "b_conn"):
            cw[k] = round_bf16(cw[k])
    return cw


# ------------------------------------------------------ CTC timestamp adapter
CTC_CLASSES = 23_863      # 23,862 tokens + blank
CTC_HEAD_DIM = 80         # 16 heads over width 1,280
CTC_FFN = 1_280


def make_ctc_weights(bf16=True, perturb=False, d=D_MODEL, dh=CTC_HEAD_DIM, ffn=CTC_FFN,
                     n_layers=2, n_classes=CTC_CLASSES, seed=WEIGHT_SEED):
    """Random-init adapter weights: upsampling taps w_conv [2, d, d] and
    b_conv [d], n_layers layer dicts (the encoder's keys, head width dh, FFN
    width ffn), lnf_g / lnf_b, projection w_out [n_classes, d], b_out.
    Draws as make_weights (N(0, 0.02^2) matrices; gains 1 / biases 0, or
    perturbed), from seeds (seed, 2000 + layer, tensor id)."""
    def tensor(layer, tid, kind, shape):
        key = (seed, 2000 + layer + 1, tid)
        if perturb and not kind.startswith("w_"):
            key = key + (1,)
        a = _draw(kind, shape, np.random.default_rng(key), perturb)
        return round_bf16(a, inplace=True) if bf16 else a

    cw = {"w_conv": tensor(-1, 0, "w_conv", (2, d, d)), "b_conv": tensor(-1, 1, "bias_d", (d,)),
          "lnf_g": tensor(-1, 2, "gain", (d,)), "lnf_b": tensor(-1, 3, "bias_d", (d,)),
          "w_out": tensor(-1, 4, "w_out", (n_classes, d)),
          "b_out": tensor(-1, 5, "bias_c", (n_classes,)), "layers": []}
    for layer in range(n_layers):
        cw["layers"].append({name: tensor(layer, tid, kind, _shape(kind, d, dh, ffn, 0))
                             for name, kind, tid in _LAYER_TENSORS})
    return cw


def alignment_case(frames, n_tokens, n_classes, seed, planted=True, repeats=0.1):
    """Synthetic CTC frame scores and a token sequence for forced alignment.

    Scores: float32 [frames, n_classes] drawn from N(-12, 2^2) (blank is the
    last class).  Tokens: n_tokens ids in 0 .. n_classes - 2, each equal to its
    predecessor with probability `repeats`.  With `planted`, one valid
    segmentation of the tokens into frames (blank runs between tokens where
    room allows, always between equal neighbours) is drawn and its classes
    get +10 in their frames, so one path stands out; the scores are not
    normalised (the alignment needs no normalisation).  Returns (scores,
    tokens)."""
    rng = np.random.default_rng(seed)
    lp = rng.normal(-12.0, 2.0, size=(frames, n_classes)).astype(np.float32)
    tokens = []
    for i in range(n_tokens):
        if i and rng.random() < repeats:
            tokens.append(tokens[-1])
        else:
            tokens.append(int(rng.integers(0, n_classes - 1)))
    if planted and n_tokens:
        blank = n_classes - 1
        need = n_tokens + sum(1 for a, b in zip(tokens, tokens[1:]) if a == b)
        if frames >= need:
            # one frame per token and one blank between equal neighbours, the
            # spare frames spread at random over tokens and blank gaps
            runs = []   # (class, length)
            for i, tk in enumerate(tokens):
                if i and tokens[i - 1] == tk:
                    runs.append([blank, 1])
                elif i:
                    runs.append([blank, 0])
                runs.append([tk, 1])
            runs = [[blank, 0]] + runs + [[blank, 0]]
            spare = frames - need
            for j in rng.integers(0, len(runs), size=spare):
                runs[int(j)][1] += 1
            t = 0
            for cls, n in runs:
                lp[t:t + n, cls] += 10.0
                t += n
    return lp, tokens
