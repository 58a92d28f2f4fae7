"""Pins of the speaker-fusion and connector oracle (CPU only).

The fusion and connector formulas are lost from the page's text; the oracle
takes the plainest reading of the prose (activity on the ASR grid, indicators
> 0.5, LayerNorm over the 8 slots, the original Transformer's sinusoid table
with the slot index as position, added to the ASR states, then one linear
map).  These tests pin that reading to closed forms, printed constants and
library routines rather than to the oracle's own formulas.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fusion
from speech_audio_encoder_amd import workloads

SIN1, COS1 = 0.8414709848078965, 0.5403023058681398      # sin(1), cos(1)
SIN3, COS3 = 0.1411200080598672, -0.9899924966004454     # sin(3), cos(3)


def test_page_figures(page_figures):
    g = page_figures
    assert fusion.N_SPEAKERS == g["speaker_slots"] == workloads.N_SPEAKERS
    assert fusion.THRESHOLD == g["speaker_threshold"]
    assert workloads.LLM_DIM == g["llm_width"]
    assert workloads.make_connector_weights(bf16=False)["speaker_scale"] == g["speaker_kernel_scale"]
    # serving windows: 500 + 50 positions at 80 ms = 40 s + 4 s; chunks 375 = 30 s
    assert g["window_core_positions"] * g["ms_per_position"] / 1000 == g["window_core_seconds_approx"]
    assert g["window_context_positions"] * g["ms_per_position"] / 1000 == g["window_context_seconds_approx"]
    assert g["chunk_seconds"] * g["positions_per_s"] == g["positions_30s"]


def test_speaker_kernel_printed_values():
    k = fusion.speaker_kernel()
    assert k.shape == (8, 1280)
    # slot 0: sin 0 = 0 on even columns, cos 0 = 1 on odd columns
    assert np.all(k[0, 0::2] == 0.0) and np.all(k[0, 1::2] == 1.0)
    # first pair has frequency 1: slot s holds (sin s, cos s)
    assert k[1, 0] == pytest.approx(SIN1, abs=1e-15) and k[1, 1] == pytest.approx(COS1, abs=1e-15)
    assert k[3, 0] == pytest.approx(SIN3, abs=1e-15) and k[3, 1] == pytest.approx(COS3, abs=1e-15)
    assert np.allclose(fusion.speaker_kernel(scale=2.5), 2.5 * k)


def test_speaker_kernel_frequencies_and_rotation():
    k = fusion.speaker_kernel()
    z = k[:, 1::2] + 1j * k[:, 0::2]            # cos + i sin per pair
    # unit pairs; slot s is slot 1 rotated s times (z_s = z_1^s)
    assert np.allclose(np.abs(z), 1.0, atol=1e-14)
    for s in range(8):
        assert np.allclose(z[s], z[1] ** s, atol=1e-12)
    # frequencies recovered from slot 1 form a geometric sequence from 1 to
    # 10000^(-1278/1280) with ratio 10000^(-2/1280)
    w = np.angle(z[1])
    assert w[0] == pytest.approx(1.0, abs=1e-15)
    assert np.allclose(np.diff(np.log(w)), -2.0 / 1280 * np.log(10000.0), atol=1e-12)
    assert w[-1] == pytest.approx(10000.0 ** (-1278 / 1280), rel=1e-12)


def test_threshold_is_strict():
    half_up = np.nextafter(np.float32(0.5), np.float32(1.0))
    a = np.array([[0.0, 0.5, half_up, 1.0, 0.49, 0.51, 0.5, 0.99]], np.float32)
    assert fusion.speaker_indicators(a).tolist() == [[0, 0, 1, 1, 0, 1, 0, 1]]


@pytest.mark.parametrize("n_active", [1, 2, 3, 8, 0])
def test_speaker_layernorm_closed_forms(n_active):
    # k of 8 slots active: mean k/8, variance k/8 (1 - k/8); an active slot
    # maps to (1 - k/8)/sqrt(var + eps), an inactive one to -(k/8)/sqrt(var + eps)
    a = np.zeros((1, 8), np.float32)
    a[0, :n_active] = 0.9
    g = np.full(8, 1.5, np.float32)
    b = np.arange(8, dtype=np.float32) * 0.1
    n = fusion.speaker_features(a, g, b)[0]
    m = n_active / 8.0
    sd = np.sqrt(m * (1 - m) + 1e-5)
    want = np.where(np.arange(8) < n_active, (1 - m) / sd, -m / sd) * 1.5 + b
    assert np.allclose(n, want, rtol=0, atol=1e-6)
    if n_active in (0, 8):                      # no spread: output is the bias
        assert np.array_equal(n, b)


def test_speaker_layernorm_matches_torch():
    rng = np.random.default_rng(3)
    a = rng.uniform(size=(200, 8)).astype(np.float32)
    g = rng.normal(1, 0.2, 8).astype(np.float32)
    b = rng.normal(0, 0.2, 8).astype(np.float32)
    ind = torch.from_numpy((a > 0.5).astype(np.float32))
    ref = torch.nn.functional.layer_norm(ind, (8,), torch.from_numpy(g), torch.from_numpy(b),
                                         eps=1e-5).numpy()
    assert np.allclose(fusion.speaker_features(a, g, b), ref, atol=1e-5)


def test_fusion_wiring_bias_picks_one_kernel_row():
    # silent activity leaves the normalised slots at the bias; a bias of e_3
    # adds exactly kernel row 3 (sin 3, cos 3, ...) to every state
    cw = workloads.make_connector_weights(bf16=False)
    cw["spk_ln_b"] = np.eye(8, dtype=np.float32)[3]
    h = np.random.default_rng(4).normal(size=(5, 1280)).astype(np.float32)
    got = fusion.fuse_speakers(h, np.zeros((5, 8), np.float32), cw) - h
    assert np.allclose(got[:, 0], SIN3, atol=1e-6) and np.allclose(got[:, 1], COS3, atol=1e-6)
    assert np.allclose(got, fusion.speaker_kernel()[3].astype(np.float32), atol=1e-6)
    cw["spk_ln_b"] = np.zeros(8, np.float32)
    assert np.array_equal(fusion.fuse_speakers(h, np.zeros((5, 8), np.float32), cw), h)


def test_fusion_matches_torch_chain():
    # LayerNorm over slots, product with the table, residual add, linear map:
    # the same chain written with torch's library routines
    cw = workloads.make_connector_weights(bf16=False, perturb=True)
    rng = np.random.default_rng(5)
    h = rng.normal(size=(37, 1280)).astype(np.float32)
    act = workloads.speaker_activity(37, seed=6)
    t = torch.from_numpy
    ind = t((act > 0.5).astype(np.float32))
    n = torch.nn.functional.layer_norm(ind, (8,), t(cw["spk_ln_g"]), t(cw["spk_ln_b"]), eps=1e-5)
    pos = torch.arange(8, dtype=torch.float64)[:, None]
    w = torch.pow(torch.tensor(10000.0, dtype=torch.float64),
                  -torch.arange(0, 1280, 2, dtype=torch.float64) / 1280)
    table = torch.stack([torch.sin(pos * w), torch.cos(pos * w)], dim=-1).reshape(8, 1280)
    fused = t(h).double() + n.double() @ table
    z = torch.nn.functional.linear(fused, t(cw["w_conn"]).double(), t(cw["b_conn"]).double())
    got = fusion.connector(fusion.fuse_speakers(h, act, cw), cw)
    assert got.shape == (37, 2688)
    assert np.allclose(got, z.numpy(), rtol=0, atol=2e-4)


def test_encode_fused_silent_is_connector_of_encoder():
    w = workloads.make_weights(1, bf16=False, perturb=True, d=256, dh=128, ffn=1024)
    cw = workloads.make_connector_weights(bf16=False, d=256, out_dim=384)
    audio, _ = workloads.custom_audio([20_000], seed=7)
    h = oracle.encode(audio[0], w)
    quiet = np.full((h.shape[0], 8), 0.2, np.float32)
    got = fusion.encode_fused(audio[0], w, quiet, cw)
    assert np.allclose(got, h @ cw["w_conn"].T + cw["b_conn"], atol=1e-5)
    # windows pass through to the windowed encoder
    gw = fusion.encode_fused(audio[0], w, quiet, cw, windows=(4, 1))
    hw = oracle.encode_windows(audio[0], w, 4, 1)
    assert np.allclose(gw, hw @ cw["w_conn"].T + cw["b_conn"], atol=1e-5)


def test_activity_generator_shape_and_range():
    a = workloads.speaker_activity(1000, seed=8)
    assert a.shape == (1000, 8) and a.dtype == np.float32
    assert a.min() >= 0.0 and a.max() <= 1.0
    ind = a > 0.5
    assert ind.any(axis=1).mean() > 0.9          # someone speaks almost always
    assert ind.sum(axis=1).max() >= 2            # some overlap or near-threshold rows
