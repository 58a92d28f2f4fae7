"""Oracle for the log-mel frontend (float64 arithmetic, float32 result).

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Follows "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
section "How audio and speakers reach the language model": 16 kHz mono input,
128 log-mel features, 25 ms Hann window, 512-point FFT, 10 ms hop, then eight
successive frames stacked into one position (about 100 frames/s down to 12.5
positions/s).  Section "How one hour fits into 65,536 positions" gives the
count D/0.08 = 12.5 D positions for D seconds, ignoring end effects.

Readings of what the page leaves open (each also listed in the design notes):
  * no dither, pre-emphasis, DC removal or feature normalisation;
  * frame t covers samples [160 t, 160 t + 400); no centre padding, so a clip
    of N samples has F = 1 + floor((N - 400) / 160) frames (0 when N < 400);
  * the Hann window is the periodic one, w[n] = 0.5 - 0.5 cos(2 pi n / 400);
  * the 400 windowed samples sit in slots 0..399 of the 512-point transform,
    zeros after; the power spectrum |X_k|^2 is taken for k = 0..256;
  * the mel bank is Slaney's (linear below 1 kHz at 200/3 Hz per mel,
    logarithmic above with step ln(6.4)/27), 128 triangles with 130 edges
    equally spaced in mel between 0 Hz and 8 kHz, triangles linear in Hz,
    peak height 1, no area normalisation;
  * the log is natural, of (mel energy + 2^-24);
  * P = ceil(F / 8) positions; position p holds frames 8p..8p+7 frame-major
    (element j*128 + m is mel m of frame 8p + j); missing tail frames are 0.
"""

import numpy as np

SAMPLE_RATE = 16000
WIN = 400                 # 25 ms at 16 kHz
HOP = 160                 # 10 ms at 16 kHz
NFFT = 512
NBINS = NFFT // 2 + 1     # 257 non-negative frequency bins
NMELS = 128
STACK = 8
LOG_GUARD = 2.0 ** -24
MAX_SAMPLES = 3600 * SAMPLE_RATE   # the one-hour recording limit


def frame_count(n_samples):
    """Number of whole 400-sample frames at a 160-sample hop (0 if too short)."""
    n = int(n_samples)
    if n < WIN:
        return 0
    return 1 + (n - WIN) // HOP


def position_count(n_frames):
    """Number of 8-frame stacks, the last one possibly partial."""
    f = int(n_frames)
    return (f + STACK - 1) // STACK


def hann_window():
    """Periodic Hann window of length 400, float64."""
    n = np.arange(WIN, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * n / WIN)


def frame_signal(x):
    """Windowed frames [F, 400] in float64 for one clip x (1-D array)."""
    x = np.asarray(x, dtype=np.float64)
    f = frame_count(x.shape[0])
    if f == 0:
        return np.zeros((0, WIN), dtype=np.float64)
    idx = np.arange(f)[:, None] * HOP + np.arange(WIN)[None, :]
    return x[idx] * hann_window()[None, :]


def _dft_basis():
    """cos and sin of 2 pi k n / 512 for n < 400, k <= 256 (float64)."""
    n = np.arange(WIN, dtype=np.int64)[:, None]
    k = np.arange(NBINS, dtype=np.int64)[None, :]
    ang = 2.0 * np.pi * ((n * k) % NFFT).astype(np.float64) / NFFT
    return np.cos(ang), np.sin(ang)


def power_spectrum(frames):
    """|X_k|^2 for k = 0..256 of the 512-point DFT of zero-padded frames.

    X_k = sum_{n<400} s[n] exp(-2 pi i k n / 512); the zero slots 400..511 add
    nothing, so the sum runs over the 400 real samples only.  A matrix product
    is the library step; everything is float64.
    """
    frames = np.asarray(frames, dtype=np.float64)
    c, s = _dft_basis()
    re = frames @ c
    im = -(frames @ s)
    return re * re + im * im


def hz_to_mel(f):
    """Slaney mel scale: linear below 1 kHz, logarithmic above."""
    f = np.asarray(f, dtype=np.float64)
    f_sp = 200.0 / 3.0
    logstep = np.log(6.4) / 27.0
    lin = f / f_sp
    with np.errstate(divide="ignore"):
        log = 1000.0 / f_sp + np.log(np.maximum(f, 1e-300) / 1000.0) / logstep
    return np.where(f < 1000.0, lin, log)


def mel_to_hz(m):
    """Inverse of hz_to_mel."""
    m = np.asarray(m, dtype=np.float64)
    f_sp = 200.0 / 3.0
    logstep = np.log(6.4) / 27.0
    m_break = 1000.0 / f_sp
    return np.where(m < m_break, m * f_sp, 1000.0 * np.exp(logstep * (m - m_break)))


def mel_filterbank():
    """Triangular mel weights W [128, 257], float64, peak 1 at each centre."""
    edges_mel = np.linspace(hz_to_mel(0.0), hz_to_mel(SAMPLE_RATE / 2.0), NMELS + 2)
    edges_hz = mel_to_hz(edges_mel)
    bin_hz = np.arange(NBINS, dtype=np.float64) * SAMPLE_RATE / NFFT
    w = np.zeros((NMELS, NBINS), dtype=np.float64)
    for m in range(NMELS):
        lo, mid, hi = edges_hz[m], edges_hz[m + 1], edges_hz[m + 2]
        rising = (bin_hz - lo) / (mid - lo)
        falling = (hi - bin_hz) / (hi - mid)
        w[m] = np.maximum(0.0, np.minimum(rising, falling))
    return w


def logmel(x, chunk=16384):
    """Log-mel features [F, 128] (float32) of one clip x."""
    x = np.asarray(x)
    f = frame_count(x.shape[0])
    out = np.zeros((f, NMELS), dtype=np.float32)
    w = mel_filterbank()
    for t0 in range(0, f, chunk):
        t1 = min(f, t0 + chunk)
        idx = np.arange(t0, t1)[:, None] * HOP + np.arange(WIN)[None, :]
        fr = np.asarray(x[idx], dtype=np.float64) * hann_window()[None, :]
        p = power_spectrum(fr)
        out[t0:t1] = np.log(p @ w.T + LOG_GUARD).astype(np.float32)
    return out


def logmel_batch(audio, lengths):
    """Batched log-mel [B, F(max length), 128] with frames t >= F_b set to 0.

    Each clip is computed alone from its first lengths[b] samples, so padding
    after a clip never reaches its features.
    """
    audio = np.asarray(audio)
    lengths = [int(n) for n in lengths]
    fmax = frame_count(max(lengths)) if lengths else 0
    out = np.zeros((len(lengths), fmax, NMELS), dtype=np.float32)
    for b, n in enumerate(lengths):
        f = frame_count(n)
        if f:
            out[b, :f] = logmel(audio[b, :n])
    return out


def stack_frames(feats):
    """Stack 8 successive frames: [F, 128] -> [ceil(F/8), 1024], zero tail."""
    feats = np.asarray(feats, dtype=np.float32)
    f = feats.shape[0]
    p = position_count(f)
    padded = np.zeros((p * STACK, NMELS), dtype=np.float32)
    padded[:f] = feats
    return padded.reshape(p, STACK * NMELS)
