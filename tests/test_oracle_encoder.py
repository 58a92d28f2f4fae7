"""Pins for the encoder oracle: library special cases, closed forms,
invariants and brute force on tiny inputs (CPU only).

Architecture per "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset
Audits", section "How audio and speakers reach the language model": width
1,280, 32 layers, ten heads, QK normalisation, rotary embeddings, FFN
expansion four, about 600M parameters.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from speech_audio_encoder_amd import workloads


def small_weights(d=256, dh=128, n_layers=1, in_dim=1024, seed=5, perturb=True):
    return workloads.make_weights(n_layers, bf16=False, perturb=perturb, d=d,
                                  dh=dh, ffn=4 * d, in_dim=in_dim, seed=seed)


# ------------------------------------------------------------ parameter count
def test_parameter_count_matches_page(page_figures):
    n = oracle.parameter_count()
    assert n == 631_009_024
    assert abs(n / page_figures["asr_params_approx"] - 1.0) < 0.06
    # the three-matrix (gated) FFN reading lands far from the page's figure
    gated = oracle.parameter_count(gated_ffn=True)
    assert gated / page_figures["asr_params_approx"] > 1.35


def test_parameter_count_matches_weight_dict():
    w = workloads.make_weights(1, bf16=False)
    total = w["w_in"].size + w["b_in"].size + w["lnf_g"].size + w["lnf_b"].size
    total += sum(a.size for a in w["layers"][0].values())
    assert total == oracle.parameter_count(n_layers=1)


# ---------------------------------------------------------------- layer norm
def test_layer_norm_against_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 1280)).astype(np.float32) * 3 + 1
    g = rng.standard_normal(1280).astype(np.float32)
    b = rng.standard_normal(1280).astype(np.float32)
    ref = F.layer_norm(torch.from_numpy(x), (1280,), torch.from_numpy(g),
                       torch.from_numpy(b), eps=1e-5).numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, g, b), ref, rtol=1e-5, atol=1e-5)


def test_layer_norm_moments_and_shift():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 128)).astype(np.float32) * 5
    y = oracle.layer_norm(x, np.ones(128), np.zeros(128))
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-6)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.var(axis=1), var / (var + 1e-5), rtol=1e-5)
    np.testing.assert_allclose(oracle.layer_norm(x + 3.5, np.ones(128), np.zeros(128)),
                               y, atol=2e-5)


# ---------------------------------------------------------------------- GELU
def test_gelu_against_torch_and_closed_forms():
    x = np.linspace(-8, 8, 1001).astype(np.float32)
    ref = F.gelu(torch.from_numpy(x), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(x), ref, rtol=1e-6, atol=1e-6)
    assert oracle.gelu(np.float32(0.0)) == 0.0
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, atol=1e-6)
    # Phi(1) = 0.8413447460685429
    assert abs(oracle.gelu(np.float32(1.0)) - 0.8413447460685429) < 1e-6


# ---------------------------------------------------------------------- RoPE
def test_rope_worked_example():
    cos, sin = oracle.rope_tables(3, 128)
    assert cos[0].tolist() == [1.0] * 64 and sin[0].tolist() == [0.0] * 64
    assert abs(cos[1, 0] - math.cos(1.0)) < 1e-7 and abs(sin[1, 0] - math.sin(1.0)) < 1e-7
    theta63 = 10000.0 ** (-63 / 64)
    assert abs(sin[2, 63] - math.sin(2 * theta63)) < 1e-9
    e0 = np.zeros((3, 128), np.float32)
    e0[:, 0] = 1.0
    r = oracle.apply_rope(e0, cos, sin)
    # position 1: e_0 -> cos(1) e_0 + sin(1) e_64
    assert abs(r[1, 0] - math.cos(1)) < 1e-6 and abs(r[1, 64] - math.sin(1)) < 1e-6
    assert np.count_nonzero(r[1]) == 2
    e64 = np.zeros((3, 128), np.float32)
    e64[:, 64] = 1.0
    r = oracle.apply_rope(e64, cos, sin)
    assert abs(r[1, 0] + math.sin(1)) < 1e-6 and abs(r[1, 64] - math.cos(1)) < 1e-6


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    cos, sin = oracle.rope_tables(50, 128)
    r = oracle.apply_rope(x, cos, sin)
    p = np.arange(50)[:, None]
    theta = 10000.0 ** (-np.arange(64) / 64.0)
    z = (x[:, :64] + 1j * x[:, 64:]).astype(np.complex128) * np.exp(1j * p * theta)
    np.testing.assert_allclose(r[:, :64], z.real, atol=2e-5)
    np.testing.assert_allclose(r[:, 64:], z.imag, atol=2e-5)
    np.testing.assert_allclose(np.linalg.norm(r, axis=1), np.linalg.norm(x, axis=1), rtol=1e-5)


def test_rope_scores_depend_on_offset_only():
    rng = np.random.default_rng(4)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)
    cos, sin = oracle.rope_tables(400, 128)

    def rot(v, p):
        return oracle.apply_rope(v[None], cos[p:p + 1], sin[p:p + 1])[0]

    base = float(rot(q, 5) @ rot(k, 2))
    for s in (1, 17, 300):
        assert abs(float(rot(q, 5 + s) @ rot(k, 2 + s)) - base) < 1e-3


# ----------------------------------------------------------------- attention
def brute_attention(q, k, v):
    t, dh = q.shape
    out = np.zeros((t, v.shape[1]))
    for i in range(t):
        s = [sum(float(q[i, c]) * float(k[j, c]) for c in range(dh)) / math.sqrt(dh)
             for j in range(t)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        for j in range(t):
            out[i] += e[j] / z * v[j].astype(np.float64)
    return out


def test_attention_brute_force():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((6, 4)).astype(np.float32) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v), brute_attention(q, k, v),
                               rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(oracle.attention(q, k, v, block=4),
                               oracle.attention(q, k, v), rtol=0, atol=1e-6)


def test_attention_against_torch_sdpa():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((300, 128)).astype(np.float32) * 2 for _ in range(3))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None]).numpy()[0]
    np.testing.assert_allclose(oracle.attention(q, k, v, block=64), ref, atol=1e-4)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, 128)).astype(np.float32)
    q = rng.standard_normal((1, 128)).astype(np.float32)
    np.testing.assert_allclose(oracle.attention(q, q, v), v, rtol=1e-6)
    v = rng.standard_normal((9, 128)).astype(np.float32)
    k = rng.standard_normal((9, 128)).astype(np.float32)
    zq = np.zeros((9, 128), np.float32)
    np.testing.assert_allclose(oracle.attention(zq, k, v), np.tile(v.mean(0), (9, 1)),
                               rtol=1e-5, atol=1e-6)


# -------------------------------------------------------------------- layers
def brute_layer(x, lw):
    """Scalar-loop reading of one layer straight from the stated layout."""
    x = x.astype(np.float64)
    t, d = x.shape
    dh = len(lw["q_g"])
    nh = d // dh

    def ln(row, g, b):
        mu = sum(row) / len(row)
        var = sum((r - mu) ** 2 for r in row) / len(row)
        return [(r - mu) / math.sqrt(var + 1e-5) * float(gg) + float(bb)
                for r, gg, bb in zip(row, g, b)]

    def lin(row, w, b):
        return [sum(float(w[o, i]) * row[i] for i in range(len(row))) + float(b[o])
                for o in range(w.shape[0])]

    def rope(vec, p):
        half = len(vec) // 2
        out = list(vec)
        for i in range(half):
            a = p * 10000.0 ** (-i / half)
            c, s = math.cos(a), math.sin(a)
            out[i] = vec[i] * c - vec[i + half] * s
            out[i + half] = vec[i + half] * c + vec[i] * s
        return out

    a = [ln(list(x[p]), lw["ln1_g"], lw["ln1_b"]) for p in range(t)]
    qkv = [lin(a[p], lw["w_qkv"], lw["b_qkv"]) for p in range(t)]
    o = [[0.0] * d for _ in range(t)]
    for h in range(nh):
        qs = [rope(ln(qkv[p][h * dh:(h + 1) * dh], lw["q_g"], lw["q_b"]), p) for p in range(t)]
        ks = [rope(ln(qkv[p][d + h * dh:d + (h + 1) * dh], lw["k_g"], lw["k_b"]), p)
              for p in range(t)]
        vs = [qkv[p][2 * d + h * dh:2 * d + (h + 1) * dh] for p in range(t)]
        for i in range(t):
            s = [sum(qs[i][c] * ks[j][c] for c in range(dh)) / math.sqrt(dh) for j in range(t)]
            m = max(s)
            e = [math.exp(z - m) for z in s]
            zs = sum(e)
            for c in range(dh):
                o[i][h * dh + c] = sum(e[j] / zs * vs[j][c] for j in range(t))
    x1 = [[x[p][c] + y for c, y in enumerate(lin(o[p], lw["w_o"], lw["b_o"]))] for p in range(t)]
    out = []
    for p in range(t):
        a2 = ln(x1[p], lw["ln2_g"], lw["ln2_b"])
        u = [0.5 * z * (1 + math.erf(z / math.sqrt(2))) for z in lin(a2, lw["w_up"], lw["b_up"])]
        out.append([x1[p][c] + y for c, y in enumerate(lin(u, lw["w_down"], lw["b_down"]))])
    return np.array(out)


def test_layer_against_scalar_brute_force():
    d, dh = 8, 4
    w = workloads.make_weights(1, bf16=False, perturb=True, d=d, dh=dh, ffn=4 * d,
                               in_dim=16, seed=11)
    lw = w["layers"][0]
    # larger weights than the default 0.02 so that attention is far from uniform
    for key in ("w_qkv", "w_o", "w_up", "w_down"):
        lw[key] = lw[key] * 40
    rng = np.random.default_rng(12)
    x = rng.standard_normal((5, d)).astype(np.float32)
    np.testing.assert_allclose(oracle.encoder_layer(x, lw), brute_layer(x, lw),
                               rtol=2e-4, atol=2e-4)


def test_single_position_layer_is_library_composition():
    # with one position attention returns v exactly, so a layer is a chain of
    # torch's linear / layer_norm / gelu
    w = small_weights()
    lw = w["layers"][0]
    d = 256
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, d)).astype(np.float32)
    T = {k: torch.from_numpy(np.asarray(v)) for k, v in lw.items()}
    xt = torch.from_numpy(x)
    a = F.layer_norm(xt, (d,), T["ln1_g"], T["ln1_b"], eps=1e-5)
    v = F.linear(a, T["w_qkv"][2 * d:], T["b_qkv"][2 * d:])
    x1 = xt + F.linear(v, T["w_o"], T["b_o"])
    a2 = F.layer_norm(x1, (d,), T["ln2_g"], T["ln2_b"], eps=1e-5)
    ref = x1 + F.linear(F.gelu(F.linear(a2, T["w_up"], T["b_up"])), T["w_down"], T["b_down"])
    np.testing.assert_allclose(oracle.encoder_layer(x, lw), ref.numpy(), rtol=1e-5, atol=1e-5)


def test_qk_norm_removes_per_head_shift():
    w = small_weights()
    lw = dict(w["layers"][0])
    rng = np.random.default_rng(14)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    base = oracle.encoder_layer(x, lw)
    b = lw["b_qkv"].copy()
    b[0:128] += 2.5          # constant on every q dim of head 0
    b[256 + 128:512] -= 1.5  # constant on every k dim of head 1
    lw["b_qkv"] = b
    np.testing.assert_allclose(oracle.encoder_layer(x, lw), base, atol=2e-4)


def test_zero_blocks_reduce_to_projection_and_norm():
    w = small_weights(n_layers=2)
    for lw in w["layers"]:
        for key in ("w_qkv", "b_qkv", "w_o", "b_o", "w_up", "b_up", "w_down", "b_down"):
            lw[key] = np.zeros_like(lw[key])
    rng = np.random.default_rng(15)
    feats = rng.standard_normal((21, 128)).astype(np.float32)
    s = torch.from_numpy(oracle.stack_frames(feats))
    ref = F.layer_norm(F.linear(s, torch.from_numpy(w["w_in"]), torch.from_numpy(w["b_in"])),
                       (256,), torch.from_numpy(w["lnf_g"]), torch.from_numpy(w["lnf_b"]),
                       eps=1e-5)
    np.testing.assert_allclose(oracle.encode_from_logmel(feats, w), ref.numpy(),
                               rtol=1e-5, atol=1e-5)


def test_encode_batch_is_per_clip():
    w = small_weights(n_layers=1)
    audio, lengths = workloads.custom_audio([5000, 300, 3210], seed=21)
    out = oracle.encode_batch(audio, lengths, w)
    assert out.shape == (3, oracle.position_count(oracle.frame_count(5000)), 256)
    for b, n in enumerate(lengths):
        e = oracle.encode(audio[b, :n], w)
        np.testing.assert_array_equal(out[b, :len(e)], e)
        assert np.all(out[b, len(e):] == 0.0)
    assert np.all(out[1] == 0.0)


def test_encoder_output_is_normalised():
    w = small_weights(n_layers=2, perturb=False)
    audio, lengths = workloads.custom_audio([9000], seed=22)
    e = oracle.encode(audio[0], w)
    np.testing.assert_allclose(e.mean(axis=1), 0.0, atol=1e-5)
    np.testing.assert_allclose(e.var(axis=1), 1.0, atol=1e-3)


def test_row_subset_matches_full_layer():
    w = small_weights(n_layers=2)
    rng = np.random.default_rng(16)
    feats = rng.standard_normal((80, 128)).astype(np.float32)
    full = oracle.encode_from_logmel(feats, w)
    rows = np.array([0, 3, 9])
    np.testing.assert_allclose(oracle.encode_from_logmel(feats, w, rows=rows), full[rows],
                               rtol=1e-5, atol=1e-5)


# ----------------------------------------------------------------- windows
def _segment(audio, st, en):
    """Audio whose frames are exactly frames 8 st .. 8 en - 1 of the clip
    (fewer at the clip's end): frame t covers samples [160 t, 160 t + 400)."""
    s0 = 160 * 8 * st
    s1 = 160 * (8 * en - 1) + 400
    return audio[s0:min(len(audio), s1)]


def test_windows_whole_clip_is_full_encoder():
    w = small_weights(n_layers=2)
    audio, _ = workloads.custom_audio([23_000], seed=71)
    x = audio[0]
    full = oracle.encode(x, w)
    assert np.array_equal(oracle.encode_windows(x, w, core=full.shape[0], context=0), full)
    assert np.array_equal(oracle.encode_windows(x, w, core=10 ** 6, context=7), full)


@pytest.mark.parametrize("core,context", [(5, 0), (4, 2), (3, 5)])
def test_windows_equal_encoder_on_audio_segments(core, context):
    # Independent route: each window's sequence re-derived from the waveform
    # (its samples cut out and encoded as a clip of its own), not from the
    # clip's features.
    w = small_weights(n_layers=2)
    audio, _ = workloads.custom_audio([31_000], seed=73)   # 193 frames, 25 positions
    x = audio[0]
    P = oracle.position_count(oracle.frame_count(len(x)))
    got = oracle.encode_windows(x, w, core, context)
    assert got.shape == (P, w["w_in"].shape[0])
    for c0 in range(0, P, core):
        st, en = max(0, c0 - context), min(P, c0 + core + context)
        ref = oracle.encode(_segment(x, st, en), w)
        assert ref.shape[0] == en - st
        c1 = min(P, c0 + core)
        np.testing.assert_allclose(got[c0:c1], ref[c0 - st:c1 - st], rtol=0, atol=1e-5)
    # windows change the result (attention scope), so a wrong scope would show
    assert not np.allclose(got, oracle.encode(x, w), atol=1e-3)
