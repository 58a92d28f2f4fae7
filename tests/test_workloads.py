"""The seeded input generators: shapes, ranges, determinism (CPU only)."""

import numpy as np

from speech_audio_encoder_amd import workloads


def test_tiny_and_clip30_shapes():
    a, n = workloads.workload_audio("tiny")
    assert a.shape == (1, 16000) and a.dtype == np.float32 and n.tolist() == [16000]
    assert np.abs(a).max() < 1.0
    a2, _ = workloads.workload_audio("tiny")
    np.testing.assert_array_equal(a, a2)


def test_batch64_lengths_and_padding():
    a, n = workloads.workload_audio("batch64")
    assert a.shape == (64, int(n.max()))
    assert n.min() >= 80_000 and n.max() <= 480_000
    for b in range(64):
        assert np.all(a[b, n[b]:] == 0.0)


def test_segment_mixture_has_quiet_and_loud_parts():
    x = workloads.segment_mixture(np.random.default_rng(4), 30 * 16000)
    rms = np.sqrt((x.reshape(-1, 1600).astype(np.float64) ** 2).mean(axis=1))
    assert rms.min() < 1e-3 and rms.max() > 0.1


def test_weights_bf16_exact_and_prefix_stable():
    w2 = workloads.make_weights(2)
    w1 = workloads.make_weights(1)
    np.testing.assert_array_equal(w2["layers"][0]["w_qkv"], w1["layers"][0]["w_qkv"])
    u = w2["layers"][1]["w_up"].view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    assert abs(float(w2["layers"][1]["w_up"].std()) - 0.02) < 1e-3
    assert np.all(w2["layers"][0]["b_qkv"] == 0) and np.all(w2["lnf_g"] == 1)
