"""Pins for the frontend oracle: page figures, closed forms, library special
cases and invariants (CPU only).

The page is "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
section "How audio and speakers reach the language model" (16 kHz, 128 mels,
25 ms Hann window, 512-point FFT, 10 ms hop, 8-frame stack) and section "How
one hour fits into 65,536 positions" (375 positions per 30 s, 45,000 per hour).
"""

import math

import numpy as np
import pytest

import oracle


# --------------------------------------------------------------- page figures
def test_constants_match_page(page_figures):
    g = page_figures
    assert oracle.SAMPLE_RATE == g["sample_rate_hz"]
    assert oracle.NMELS == g["n_mels"]
    assert oracle.WIN == g["window_ms"] * g["sample_rate_hz"] / 1000
    assert oracle.HOP == g["hop_ms"] * g["sample_rate_hz"] / 1000
    assert oracle.NFFT == g["fft_points"]
    assert oracle.STACK == g["stack_frames"]
    assert oracle.MAX_SAMPLES == g["max_duration_s"] * g["sample_rate_hz"]


def test_position_counts_match_page(page_figures):
    g = page_figures
    sr = oracle.SAMPLE_RATE
    p30 = oracle.position_count(oracle.frame_count(30 * sr))
    p1h = oracle.position_count(oracle.frame_count(3600 * sr))
    assert p30 == g["positions_30s"]
    assert p1h == g["positions_1h"]
    # rates over a long clip: ~100 frames/s, 12.5 positions/s, 80 ms/position
    n = 3600 * sr
    f = oracle.frame_count(n)
    assert abs(f / 3600 - g["frames_per_s_approx"]) < 0.01
    assert abs(oracle.position_count(f) / 3600 - g["positions_per_s"]) < 1e-9
    assert abs(1000 * 3600 / oracle.position_count(f) - g["ms_per_position"]) < 1e-9


def test_hour_of_float32_audio_bytes(page_figures):
    assert oracle.MAX_SAMPLES * 4 == page_figures["float32_bytes_per_hour"]
    assert oracle.MAX_SAMPLES * 2 == page_figures["pcm16_bytes_per_hour"]


@pytest.mark.parametrize("n,f,p", [
    (0, 0, 0), (399, 0, 0), (400, 1, 1), (559, 1, 1), (560, 2, 1),
    (400 + 7 * 160, 8, 1), (400 + 8 * 160, 9, 2),
    (16_000, 98, 13), (480_000, 2_998, 375),
    (9_600_000, 59_998, 7_500), (57_600_000, 359_998, 45_000),
])
def test_frame_and_position_closed_form(n, f, p):
    assert oracle.frame_count(n) == f
    assert oracle.position_count(f) == p


# --------------------------------------------------------------------- window
def test_periodic_hann_sums():
    w = oracle.hann_window()
    assert w.shape == (400,)
    assert abs(w.sum() - 200.0) < 1e-10
    assert abs((w * w).sum() - 150.0) < 1e-10
    assert w[0] == 0.0 and abs(w[200] - 1.0) < 1e-15


def test_constant_signal_dc_bin():
    c = 0.37
    fr = oracle.frame_signal(np.full(400, c))
    p = oracle.power_spectrum(fr)[0]
    assert abs(p[0] - (200.0 * c) ** 2) < 1e-9


def test_frame_signal_positions():
    x = np.arange(1000, dtype=np.float64)
    fr = oracle.frame_signal(x)
    assert fr.shape == (oracle.frame_count(1000), 400)
    w = oracle.hann_window()
    np.testing.assert_array_equal(fr[2], x[320:720] * w)


# ------------------------------------------------------------------ transform
def test_dft_matches_numpy_rfft():
    rng = np.random.default_rng(7)
    fr = rng.standard_normal((16, 400))
    ref = np.abs(np.fft.rfft(fr, n=512, axis=-1)) ** 2
    got = oracle.power_spectrum(fr)
    assert got.shape == (16, 257)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-10 * ref.max())


def test_parseval():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((5, 400))
    p = oracle.power_spectrum(s)
    total = p[:, 0] + 2.0 * p[:, 1:256].sum(axis=1) + p[:, 256]
    np.testing.assert_allclose(total, 512.0 * (s * s).sum(axis=1), rtol=1e-12)


@pytest.mark.parametrize("k0,amp,phase", [(3, 0.3, 0.1), (40, 0.1, 1.3),
                                          (128, 0.25, 2.0), (253, 0.2, 4.0)])
def test_bin_centred_tone(k0, amp, phase):
    n = np.arange(400)
    x = amp * np.sin(2 * np.pi * k0 * n / 512 + phase)
    p = oracle.power_spectrum(oracle.frame_signal(x))[0]
    assert int(np.argmax(p)) == k0
    assert abs(p[k0] / (100.0 * amp) ** 2 - 1.0) < 0.02


def test_white_noise_mean_power():
    sigma = 0.05
    rng = np.random.default_rng(9)
    x = sigma * rng.standard_normal(400 + 4999 * 160)
    p = oracle.power_spectrum(oracle.frame_signal(x))
    mean = p[:, 1:256].mean()
    assert abs(mean / (150.0 * sigma ** 2) - 1.0) < 0.02
    per_bin = p[:, 1:256].mean(axis=0) / (150.0 * sigma ** 2)
    assert np.all(np.abs(per_bin - 1.0) < 0.15)


# ------------------------------------------------------------------ mel scale
def test_slaney_scale_closed_forms():
    assert abs(oracle.hz_to_mel(1000.0) - 15.0) < 1e-12
    assert abs(oracle.hz_to_mel(500.0) - 7.5) < 1e-12
    assert abs(oracle.hz_to_mel(6400.0) - 42.0) < 1e-12       # 27 log steps above 1 kHz
    assert abs(oracle.hz_to_mel(8000.0) - (15 + 27 * math.log(8) / math.log(6.4))) < 1e-12
    assert abs(oracle.hz_to_mel(8000.0) - 45.2456) < 1e-4
    f = np.array([0.0, 10.0, 999.0, 1000.0, 1234.5, 7999.0])
    np.testing.assert_allclose(oracle.mel_to_hz(oracle.hz_to_mel(f)), f, rtol=1e-12, atol=1e-12)


def test_mel_filterbank_structure():
    w = oracle.mel_filterbank()
    assert w.shape == (128, 257)
    assert np.all(w >= 0.0) and np.all(w <= 1.0 + 1e-12)
    assert np.all((w > 0).sum(axis=1) >= 1)            # every band sees a bin
    assert np.all(w[:, 0] == 0.0) and np.all(w[:, 256] == 0.0)
    assert np.all(w[:, 1:256].sum(axis=0) > 0.0)        # bins 1..255 all covered
    # bands are ordered: first nonzero bin never decreases with m
    first = np.argmax(w > 0, axis=1)
    assert np.all(np.diff(first) >= 0)


def test_mel_partition_of_unity():
    w = oracle.mel_filterbank()
    edges = oracle.mel_to_hz(np.linspace(0.0, oracle.hz_to_mel(8000.0), 130))
    bin_hz = np.arange(257) * 16000.0 / 512
    inside = (bin_hz >= edges[1]) & (bin_hz <= edges[128])
    np.testing.assert_allclose(w[:, inside].sum(axis=0), 1.0, atol=1e-12)


# ------------------------------------------------------------------- log-mel
def test_logmel_silence_floor():
    feats = oracle.logmel(np.zeros(16000, dtype=np.float32))
    assert feats.shape == (98, 128)
    np.testing.assert_allclose(feats, math.log(2.0 ** -24), rtol=0, atol=1e-6)
    assert abs(math.log(2.0 ** -24) + 16.6355) < 1e-4


def test_logmel_matches_library_pipeline():
    # independent route: numpy's FFT of a periodic-Hann frame, then the bank
    rng = np.random.default_rng(10)
    x = (0.1 * rng.standard_normal(5000)).astype(np.float32)
    f = oracle.frame_count(len(x))
    n = np.arange(400)
    win = np.sin(np.pi * n / 400) ** 2                  # = periodic Hann
    fr = np.stack([x[160 * t:160 * t + 400].astype(np.float64) * win for t in range(f)])
    spec = np.abs(np.fft.rfft(fr, n=512, axis=-1)) ** 2
    ref = np.log(spec @ oracle.mel_filterbank().T + 2.0 ** -24)
    np.testing.assert_allclose(oracle.logmel(x), ref, rtol=0, atol=2e-6)


def test_logmel_short_and_chunked():
    assert oracle.logmel(np.zeros(399, np.float32)).shape == (0, 128)
    rng = np.random.default_rng(11)
    x = rng.standard_normal(400 + 99 * 160).astype(np.float32)
    a = oracle.logmel(x)
    b = oracle.logmel(x, chunk=7)
    np.testing.assert_array_equal(a, b)


def test_logmel_batch_padding_independent():
    rng = np.random.default_rng(12)
    lengths = [1000, 399, 2345]
    audio = rng.standard_normal((3, 2345)).astype(np.float32)
    out = oracle.logmel_batch(audio, lengths)
    assert out.shape == (3, oracle.frame_count(2345), 128)
    garbage = audio.copy()
    garbage[0, 1000:] = 1e6
    garbage[1, 399:] = -1e6
    out2 = oracle.logmel_batch(garbage, lengths)
    np.testing.assert_array_equal(out, out2)
    assert np.all(out[0, oracle.frame_count(1000):] == 0.0)
    assert np.all(out[1] == 0.0)
    np.testing.assert_array_equal(out[2], oracle.logmel(audio[2]))


# --------------------------------------------------------------------- stack
def test_stack_frames_gather_and_tail():
    feats = np.arange(98 * 128, dtype=np.float32).reshape(98, 128)
    s = oracle.stack_frames(feats)
    assert s.shape == (13, 1024)
    for p in range(13):
        for j in range(8):
            t = 8 * p + j
            row = s[p, j * 128:(j + 1) * 128]
            if t < 98:
                np.testing.assert_array_equal(row, feats[t])
            else:
                assert np.all(row == 0.0)
    # last position: 2 real frames, 6 zero frames
    assert np.all(s[12, 256:] == 0.0) and np.any(s[12, :256] != 0.0)
