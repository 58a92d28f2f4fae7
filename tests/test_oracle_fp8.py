"""Pins of the FP8 (E4M3, per-tensor scales) oracle, CPU only.

The E4M3 rounding is pinned to the format's definition (OCP FP8: bias 7, 3
mantissa bits, largest finite 448, subnormals down to 2^-9) by brute force
over its value grid; the quantized linear map reduces to the plain linear map
when every operand is on the grid; the FP8 layer's structure is pinned to the
unquantized layer through its calibration mode.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from speech_audio_encoder_amd import workloads


def e4m3_grid():
    """Every finite non-negative E4M3 value with its mantissa bits, from the
    format definition."""
    vals, mant = [0.0], [0]
    for m in range(1, 8):                        # subnormals m/8 * 2^-6
        vals.append(m / 8 * 2.0 ** -6)
        mant.append(m)
    for e in range(1, 16):                       # normals (1 + m/8) 2^(e-7)
        for m in range(8):
            if e == 15 and m == 7:               # the NaN code
                continue
            vals.append((1 + m / 8) * 2.0 ** (e - 7))
            mant.append(m)
    return np.array(vals), np.array(mant)


def test_grid_landmarks():
    g, _ = e4m3_grid()
    assert g.max() == 448.0 and g[g > 0].min() == 2.0 ** -9
    assert 2.0 ** -6 in g and len(g) == 127
    assert np.array_equal(fp8.e4m3(g.astype(np.float32)), g)
    assert np.array_equal(fp8.e4m3(-g.astype(np.float32)), -g)


def test_rounding_is_nearest_ties_to_even_brute_force():
    g, mant = e4m3_grid()
    rng = np.random.default_rng(0)
    mids = (g[1:] + g[:-1]) / 2
    xs = np.concatenate([rng.uniform(0, 448, 20000), rng.uniform(0, 0.05, 20000), mids,
                         np.nextafter(mids.astype(np.float32), np.float32(0)),
                         np.nextafter(mids.astype(np.float32), np.float32(1000))]).astype(np.float32)
    got = fp8.e4m3(xs)
    for x, y in zip(xs.astype(np.float64), got.astype(np.float64)):
        d = np.abs(g - x)
        best = np.nonzero(d == d.min())[0]
        if len(best) == 1:
            assert y == g[best[0]], (x, y)
        else:                                    # a tie: the even mantissa wins
            even = [i for i in best if mant[i] % 2 == 0]
            assert len(even) == 1 and y == g[even[0]], (x, y)


def test_saturation_and_sign():
    x = np.array([448.0, 449.0, 464.0, 500.0, 1e30, -1e30, -470.0], np.float32)
    assert fp8.e4m3(x).tolist() == [448, 448, 448, 448, 448, -448, -448]


def test_quantize_with_power_of_two_scale_is_exact_on_grid():
    g, _ = e4m3_grid()
    v = np.concatenate([g, -g]).astype(np.float32) * np.float32(0.25)
    assert np.array_equal(fp8.quantize(v, 0.25), np.concatenate([g, -g]))


def test_weight_scale_and_zero_matrix():
    w = np.array([[0.5, -2.0], [1.0, 0.25]], np.float32)
    assert fp8.weight_scale(w) == np.float32(2.0) / np.float32(448)
    assert fp8.weight_scale(np.zeros((3, 3), np.float32)) == 1.0
    q, s = fp8.quantize_weight(w)
    assert np.abs(q).max() == 448.0 and s == np.float32(2.0) / np.float32(448)
    assert np.array_equal(fp8.scales_from_amax([[0.0, 896.0]]), np.float32([[1.0, 2.0]]))


def test_linear_fp8_reduces_to_linear_on_grid():
    # operands already on the E4M3 grid under power-of-two scales: the FP8
    # map is the plain linear map (torch's)
    g, _ = e4m3_grid()
    rng = np.random.default_rng(1)
    pick = g[(g > 0.01) & (g < 100)]
    x = (rng.choice(pick, (7, 64)) * rng.choice([-1, 1], (7, 64))).astype(np.float32) * 0.5
    wq = (rng.choice(pick, (48, 64)) * rng.choice([-1, 1], (48, 64))).astype(np.float32)
    b = rng.normal(size=48).astype(np.float32)
    got = fp8.linear_fp8(x, wq, np.float32(0.125), b, np.float32(0.5))
    ref = torch.nn.functional.linear(torch.from_numpy(x).double(),
                                     torch.from_numpy(wq * 0.125).double(),
                                     torch.from_numpy(b).double()).numpy()
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-5)


def small_weights():
    return workloads.make_weights(2, bf16=False, perturb=True, d=256, dh=128, ffn=1024)


def test_calibration_mode_is_the_unquantized_layer():
    w = small_weights()
    x = np.random.default_rng(2).normal(size=(19, 256)).astype(np.float32)
    rec = []
    got = fp8.encoder_layer_fp8(x, w["layers"][0], None, None, record=rec)
    assert np.allclose(got, oracle.encoder_layer(x, w["layers"][0]), atol=1e-5)
    t = torch.from_numpy(x)
    ln1 = torch.nn.functional.layer_norm(t, (256,), torch.from_numpy(w["layers"][0]["ln1_g"]),
                                         torch.from_numpy(w["layers"][0]["ln1_b"]), eps=1e-5)
    assert len(rec) == 4 and rec[0] == pytest.approx(float(ln1.abs().max()), rel=1e-5)
    assert all(r > 0 for r in rec)


def test_fp8_encoder_close_to_unquantized_and_calibration():
    w = small_weights()
    audio, _ = workloads.custom_audio([24_000, 9_000], seed=3)
    clips = [audio[0], audio[1, :9_000]]
    amax = fp8.calibrate(clips, w)
    assert amax.shape == (2, 4) and np.all(amax > 0)
    scales = fp8.scales_from_amax(amax)
    ref = oracle.encode(clips[0], w)
    got = fp8.encode_fp8(clips[0], w, scales)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert 1e-4 < rel < 0.15      # quantized, but close
    # scales far too small saturate everything: a different result
    bad = fp8.encode_fp8(clips[0], w, scales * 1e-3)
    assert np.abs(bad - ref).max() > 3 * np.abs(got - ref).max()
    assert fp8.encode_fp8(np.zeros(300, np.float32), w, scales).shape == (0, 256)


# ------------------------------------------------------------------
# The FP8 layer against a torch layer that casts through float8_e4m3fn at
# exactly the four stated points (the inputs of the QKV, output, FFN-up and
# FFN-down maps), with weight codes from the definition (bf16 value, scale
# amax / 448, codes of w * fp32(1 / s_w)).  Input scales are powers of two,
# so a value's code is the torch cast of value / s exactly; each map gets a
# different scale chosen so that value / s reaches [224, 448) at the
# largest input, and the wrong scale for a map saturates its top values or
# coarsens its small ones.
F = torch.nn.functional


def _pin_weights():
    w = workloads.make_weights(1, bf16=False, perturb=True, d=64, dh=16, ffn=256)
    lw = w["layers"][0]
    lw["ln1_g"] = lw["ln1_g"] * np.float32(0.4)     # LN1 output narrower than the GELU output
    lw["ln2_g"] = lw["ln2_g"] * np.float32(6.0)     # LN2 output wider than both
    lw["w_down"] = lw["w_down"] * np.float32(4.0)
    return lw


def _torch_fp8_layer(x, lw, scales, quantize_at=("qkv", "o", "up", "down")):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))  # noqa: E731
    d = x.shape[1]
    dh = len(lw["q_g"])

    def qdq(v, s):
        return (v / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).to(torch.float32)

    def lin8(v, wname, bname, s_x, point):
        wb = t(lw[wname]).to(torch.bfloat16).to(torch.float32)
        s_w = wb.abs().max() / torch.tensor(448.0)
        codes = (wb * (torch.tensor(1.0) / s_w)).clamp(-448.0, 448.0)
        codes = codes.to(torch.float8_e4m3fn).to(torch.float64)
        if point in quantize_at:
            acc = qdq(v, s_x).double() @ codes.T
            alpha = (torch.tensor(s_x, dtype=torch.float32) * s_w).double()
            return (acc * alpha).float() + t(lw[bname])
        return F.linear(v, t(lw[wname]), t(lw[bname]))

    xt = t(x)
    h = F.layer_norm(xt, (d,), t(lw["ln1_g"]), t(lw["ln1_b"]), eps=1e-5)
    qkv = lin8(h, "w_qkv", "b_qkv", scales[0], "qkv")
    n = x.shape[0]
    ang = torch.arange(n, dtype=torch.float64)[:, None] * \
        10000.0 ** (-torch.arange(dh // 2, dtype=torch.float64) / (dh // 2))
    rot = torch.polar(torch.ones_like(ang), ang).to(torch.complex64)

    def norm_rot(v, g, b):
        v = F.layer_norm(v, (dh,), t(lw[g]), t(lw[b]), eps=1e-5)
        z = torch.complex(v[:, :dh // 2], v[:, dh // 2:]) * rot
        return torch.cat([z.real, z.imag], dim=1)

    heads = []
    for hh in range(d // dh):
        q = norm_rot(qkv[:, hh * dh:(hh + 1) * dh], "q_g", "q_b")
        k = norm_rot(qkv[:, d + hh * dh:d + (hh + 1) * dh], "k_g", "k_b")
        v = qkv[:, 2 * d + hh * dh:2 * d + (hh + 1) * dh]
        heads.append(F.scaled_dot_product_attention(q[None], k[None], v[None])[0])
    o = torch.cat(heads, dim=1)
    if "o_out" in quantize_at:     # a mistake the pin must catch: quantize the output
        x1 = xt + qdq(lin8(o, "w_o", "b_o", scales[1], "none"), scales[1])
    else:
        x1 = xt + lin8(o, "w_o", "b_o", scales[1], "o")
    h2 = F.layer_norm(x1, (d,), t(lw["ln2_g"]), t(lw["ln2_b"]), eps=1e-5)
    u = F.gelu(lin8(h2, "w_up", "b_up", scales[2], "up"))
    return (x1 + lin8(u, "w_down", "b_down", scales[3], "down")).numpy()


def _pin_case():
    lw = _pin_weights()
    x = (3.0 * np.random.default_rng(12).normal(size=(11, 64))).astype(np.float32)
    rec = []
    fp8.encoder_layer_fp8(x, lw, None, None, record=rec)
    scales = [np.float32(2.0 ** np.floor(np.log2(a / 224.0))) for a in rec]
    return lw, x, scales, rec


def test_fp8_layer_casts_exactly_at_the_four_map_inputs():
    lw, x, scales, rec = _pin_case()
    ratios = [a / s for a, s in zip(rec, scales)]
    assert all(224.0 <= r < 448.0 for r in ratios), ratios
    assert len(set(float(s) for s in scales)) == 4, scales      # one scale per map
    qw = fp8.prepare_fp8({"layers": [lw]})[0]
    got = fp8.encoder_layer_fp8(x, lw, qw, scales)
    ref = _torch_fp8_layer(x, lw, scales)
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() <= 1e-5 * scale
    # against the unquantized layer the difference is quantization-sized
    plain = oracle.encoder_layer(x, lw)
    assert np.abs(got - plain).max() > 1e-3 * scale


@pytest.mark.parametrize("mistake", ["swap_qkv_up", "swap_o_down", "no_quant_o",
                                     "quantize_o_output", "no_quant_down"])
def test_fp8_layer_pin_rejects_plausible_mistakes(mistake):
    # The torch reference with one plausible mistake (a scale index swapped,
    # a map left unquantized, the output of w_o quantized instead of its
    # input) lands far outside the tolerance the oracle meets above.
    lw, x, scales, _ = _pin_case()
    qw = fp8.prepare_fp8({"layers": [lw]})[0]
    got = fp8.encoder_layer_fp8(x, lw, qw, scales)
    s = list(scales)
    points = ("qkv", "o", "up", "down")
    if mistake == "swap_qkv_up":
        s[0], s[2] = s[2], s[0]
    elif mistake == "swap_o_down":
        s[1], s[3] = s[3], s[1]
    elif mistake == "no_quant_o":
        points = ("qkv", "up", "down")
    elif mistake == "quantize_o_output":
        points = ("qkv", "o_out", "up", "down")
    elif mistake == "no_quant_down":
        points = ("qkv", "o", "up")
    wrong = _torch_fp8_layer(x, lw, s, points)
    assert np.abs(got - wrong).max() > 100 * 1e-5 * np.abs(got).max()
