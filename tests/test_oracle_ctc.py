"""Pins of the CTC timestamp adapter oracle (CPU only)."""

import numpy as np
import torch

import oracle
from oracle import ctc
from speech_audio_encoder_amd import workloads


def small_ctc(d=160, dh=80, ffn=160, n_classes=300, perturb=True):
    return workloads.make_ctc_weights(bf16=False, perturb=perturb, d=d, dh=dh, ffn=ffn,
                                      n_classes=n_classes)


def test_parameter_count_matches_page(page_figures):
    # the page: "approximately 50M"; expansion 4 would not fit
    n = ctc.parameter_count()
    assert abs(n / page_figures["ctc_adapter_params_approx"] - 1) < 0.1
    assert ctc.parameter_count(ffn=4 * 1280) / page_figures["ctc_adapter_params_approx"] > 1.4
    assert ctc.N_CLASSES == page_figures["ctc_vocab"] + 1 == workloads.CTC_CLASSES
    cw = workloads.make_ctc_weights(bf16=False)
    counted = sum(np.asarray(v).size for k, v in cw.items() if k != "layers") + \
        sum(np.asarray(v).size for lw in cw["layers"] for v in lw.values())
    assert counted == n


def test_upsample_matches_torch_conv_transpose():
    rng = np.random.default_rng(0)
    h = rng.normal(size=(7, 24)).astype(np.float32)
    w = rng.normal(size=(2, 16, 24)).astype(np.float32)     # [tap, out, in]
    b = rng.normal(size=16).astype(np.float32)
    # torch's ConvTranspose1d weight is [in, out, kernel]
    wt = torch.from_numpy(np.ascontiguousarray(w.transpose(2, 1, 0)))
    ref = torch.nn.functional.conv_transpose1d(torch.from_numpy(h.T[None]), wt,
                                               torch.from_numpy(b), stride=2)[0].numpy().T
    got = ctc.upsample(h, w, b)
    assert got.shape == (14, 16)
    assert np.allclose(got, ref, atol=1e-5)


def test_log_softmax_matches_torch_and_normalises():
    z = np.random.default_rng(1).normal(0, 5, (9, 300)).astype(np.float32)
    got = ctc.log_softmax(z)
    assert np.allclose(got, torch.log_softmax(torch.from_numpy(z).double(), -1).numpy(), atol=1e-6)
    assert np.allclose(np.exp(got.astype(np.float64)).sum(axis=1), 1.0, atol=1e-6)


def test_adapter_layers_use_head_width_80():
    # 16 heads of 80 at width 1280: the layer oracle derives the head count
    # from q_g; the rotation at head width 80 turns pairs (i, i + 40) by
    # p * 10000^(-i/40), i.e. multiplies x_i + i x_{i+40} by exp(i p w_i)
    cw = workloads.make_ctc_weights(bf16=False, n_classes=8)
    lw = cw["layers"][0]
    assert lw["q_g"].shape == (80,) and lw["w_up"].shape == (1280, 1280)
    assert lw["w_qkv"].shape == (3840, 1280)
    cos, sin = oracle.rope_tables(50, 80)
    x = np.random.default_rng(2).normal(size=(50, 80)).astype(np.float32)
    got = oracle.apply_rope(x, cos, sin)
    z = (x[:, :40] + 1j * x[:, 40:]) * np.exp(
        1j * np.arange(50)[:, None] * 10000.0 ** (-np.arange(40) / 40))
    assert np.allclose(got, np.concatenate([z.real, z.imag], axis=1), atol=1e-4)
    y = oracle.encoder_layer(np.random.default_rng(5).normal(size=(9, 1280)).astype(np.float32),
                             lw)
    assert y.shape == (9, 1280) and np.all(np.isfinite(y))


def test_adapter_shape_and_probabilities():
    cw = small_ctc()
    h = np.random.default_rng(3).normal(size=(6, 160)).astype(np.float32)
    lp = ctc.adapter_from_states(h, cw)
    assert lp.shape == (12, 300)
    assert np.allclose(np.exp(lp.astype(np.float64)).sum(axis=1), 1.0, atol=1e-5)
    assert np.all(lp <= 0)


def test_upsampled_frames_are_independent_per_tap():
    # frame 2t + j depends on H[t] only (kernel 2, stride 2: no overlap)
    rng = np.random.default_rng(4)
    w = rng.normal(size=(2, 8, 8)).astype(np.float32)
    b = np.zeros(8, np.float32)
    h = rng.normal(size=(5, 8)).astype(np.float32)
    base = ctc.upsample(h, w, b)
    h2 = h.copy()
    h2[2] += 1.0
    diff = np.abs(ctc.upsample(h2, w, b) - base).max(axis=1)
    assert np.nonzero(diff)[0].tolist() == [4, 5]


def test_adapter_chain_with_constant_layers_matches_torch():
    # With every matrix of a layer zero, the attention branch returns its
    # output bias and the FFN branch its output bias, so layer l adds the
    # constant c_l = b_o + b_down.  The adapter is then the composition
    #   log_softmax(linear(layer_norm(conv_transpose1d(H) + c_1 + c_2)))
    # of torch routines: a dropped or misplaced final LayerNorm, a layer
    # before the upsampling, or a missing projection bias all change it.
    rng = np.random.default_rng(11)
    cw = small_ctc(n_classes=37)
    for lw in cw["layers"]:
        for name in ("w_qkv", "w_o", "w_up", "w_down"):
            lw[name] = np.zeros_like(lw[name])
        lw["b_o"] = rng.normal(0, 2.0, lw["b_o"].shape).astype(np.float32)
        lw["b_down"] = rng.normal(0, 2.0, lw["b_down"].shape).astype(np.float32)
    cw["b_out"] = rng.normal(0, 1.0, cw["b_out"].shape).astype(np.float32)
    cw["w_out"] = rng.normal(0, 0.5, cw["w_out"].shape).astype(np.float32)
    h = rng.normal(size=(6, 160)).astype(np.float32)
    F = torch.nn.functional
    t = torch.from_numpy
    wt = t(np.ascontiguousarray(cw["w_conv"].transpose(2, 1, 0))).double()   # [in, out, k]
    x = F.conv_transpose1d(t(h.T[None]).double(), wt, t(cw["b_conv"]).double(), stride=2)[0].T
    for lw in cw["layers"]:
        x = x + t(lw["b_o"]).double() + t(lw["b_down"]).double()
    x = F.layer_norm(x, (160,), t(cw["lnf_g"]).double(), t(cw["lnf_b"]).double(), eps=1e-5)
    ref = torch.log_softmax(F.linear(x, t(cw["w_out"]).double(), t(cw["b_out"]).double()), -1)
    got = ctc.adapter_from_states(h, cw)
    assert got.shape == (12, 37)
    np.testing.assert_allclose(got, ref.numpy(), atol=2e-4)
    # the pin is sensitive to where the final LayerNorm sits: applied before
    # the second layer instead, the result moves far outside the tolerance
    y = F.conv_transpose1d(t(h.T[None]).double(), wt, t(cw["b_conv"]).double(), stride=2)[0].T
    y = y + t(cw["layers"][0]["b_o"]).double() + t(cw["layers"][0]["b_down"]).double()
    y = F.layer_norm(y, (160,), t(cw["lnf_g"]).double(), t(cw["lnf_b"]).double(), eps=1e-5)
    y = y + t(cw["layers"][1]["b_o"]).double() + t(cw["layers"][1]["b_down"]).double()
    wrong = torch.log_softmax(F.linear(y, t(cw["w_out"]).double(), t(cw["b_out"]).double()), -1)
    assert np.abs(wrong.numpy() - got).max() > 0.1
