"""Oracle for the FP8 variant of the encoder (per-tensor E4M3 linear maps).

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

The nemotron-transcribe skill page (decimal.ai), section "Precision
selection", says the FP8 release is a ModelOpt export whose audio encoder is
quantized; "Nemotron 3.5 Transcribe: From Recorded Speech to Dataset Audits",
section "The long-audio memory budget is not just the KV cache", adds that the
ASR projections are kept in FP8 even in the NVFP4 mix.  Nothing more is
given; this oracle takes the plainest reading, the per-tensor FP8 scheme
(listed in the design notes as well):
  * the four linear maps of every layer (QKV, attention output, FFN up, FFN
    down) run on E4M3 codes (OCP FP8: 1 sign, 4 exponent bits with bias 7,
    3 mantissa bits, largest finite value 448, no infinities);
  * a weight matrix W (taken as its bf16 value, the precision the encoder
    stores) has one scale s_w = amax|W| / 448 (1 if W is all zero);
  * an input X has one static scale s_x per linear map, from calibration:
    s_x = amax|X| / 448 over a calibration batch of the unquantized model;
  * codes: q = RNE_e4m3(clamp(v * r, -448, 448)) with r = fp32(1 / s) and
    round-to-nearest-even onto the E4M3 grid;
  * y = (q_x . q_w) * fp32(s_x * s_w) + b, accumulated exactly here (float64)
    and in fp32 on the GPU;
  * the input projection, attention itself, the norms and the rotation stay
    as in the unquantized encoder oracle (float32 operands).
The pages fix no operand precision outside the four quantized maps, so none
is emulated.  ``operand`` (default: none) lets a caller apply a map to the
attention operands (q, k, v) and to the input projection's operands; it is
used only to measure how far a change of their precision moves the FP8
result, since every E4M3 code is a rounding decision that any upstream
difference can flip.
"""

import numpy as np
import torch

from .encoder import (apply_rope, attention, gelu, layer_norm, linear, rope_tables)
from .frontend import logmel, stack_frames

E4M3_MAX = 448.0


def round_bf16(a):
    """Nearest bfloat16 value (ties to even) of float32 a, as float32."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def e4m3(v):
    """Round float32 v to the nearest E4M3 value, ties to even, saturating at
    +-448 (the clamp comes first, so nothing rounds past the largest value)."""
    v = np.clip(np.asarray(v, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    return torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float32).numpy()


def quantize(v, s):
    """E4M3 codes (as their float values) of v under scale s: e4m3(v * (1/s))."""
    r = np.float32(1.0) / np.float32(s)
    return e4m3(np.asarray(v, dtype=np.float32) * r)


def weight_scale(w):
    amax = np.float32(np.abs(w).max()) if w.size else np.float32(0)
    return np.float32(1.0) if amax == 0 else amax / np.float32(E4M3_MAX)


def quantize_weight(w):
    """(codes, s_w) of a weight matrix, from its bf16 value."""
    wb = round_bf16(w)
    s = weight_scale(wb)
    return quantize(wb, s), s


def linear_fp8(x, wq, s_w, b, s_x):
    """y = (q(x) . wq^T) * fp32(s_x * s_w) + b."""
    xq = quantize(x, s_x).astype(np.float64)
    acc = xq @ np.asarray(wq, dtype=np.float64).T
    alpha = np.float32(np.float32(s_x) * np.float32(s_w))
    return (acc * np.float64(alpha)).astype(np.float32) + np.asarray(b, dtype=np.float32)


LINEARS = ("w_qkv", "w_o", "w_up", "w_down")


def prepare_fp8(weights):
    """Per layer: codes and scales of the four quantized matrices."""
    out = []
    for lw in weights["layers"]:
        out.append({name: quantize_weight(lw[name]) for name in LINEARS})
    return out


def encoder_layer_fp8(x, lw, qw, scales, record=None, operand=None):
    """One pre-norm block with FP8 linear maps; scales = input scales of
    (QKV, O, up, down).  record: a list that receives the amax of the four
    linear inputs (calibration), in which case the layer runs unquantized.
    operand: optional map applied to q, k, v (measurement of precision
    spread only; None leaves them as computed)."""
    d = x.shape[1]
    dh = lw["q_g"].shape[0]
    nh = d // dh

    def lin(inp, i, name, bname):
        if record is not None:
            record.append(float(np.abs(inp).max()) if inp.size else 0.0)
            return linear(inp, lw[name], lw[bname])
        wq, s_w = qw[name]
        return linear_fp8(inp, wq, s_w, lw[bname], scales[i])

    op = (lambda t: t) if operand is None else operand
    h = layer_norm(x, lw["ln1_g"], lw["ln1_b"])
    qkv = op(lin(h, 0, "w_qkv", "b_qkv"))
    cos, sin = rope_tables(x.shape[0], dh)
    heads = []
    for hh in range(nh):
        q = qkv[:, hh * dh:(hh + 1) * dh]
        k = qkv[:, d + hh * dh:d + (hh + 1) * dh]
        v = qkv[:, 2 * d + hh * dh:2 * d + (hh + 1) * dh]
        q = op(apply_rope(layer_norm(q, lw["q_g"], lw["q_b"]), cos, sin))
        k = op(apply_rope(layer_norm(k, lw["k_g"], lw["k_b"]), cos, sin))
        heads.append(attention(q, k, v))
    o = np.concatenate(heads, axis=1)
    x = x + lin(o, 1, "w_o", "b_o")
    h = layer_norm(x, lw["ln2_g"], lw["ln2_b"])
    u = gelu(lin(h, 2, "w_up", "b_up"))
    return x + lin(u, 3, "w_down", "b_down")


def _stacked_input(x, weights, operand=None):
    """Input projection (unquantized), optionally on mapped operands."""
    op = (lambda t: t) if operand is None else operand
    feats = op(stack_frames(logmel(x)))
    return linear(feats, op(weights["w_in"]), weights["b_in"])


def encode_fp8(x, weights, input_scales, n_layers=None, qw=None, operand=None):
    """Waveform of one clip -> embeddings [P, d] with FP8 linear maps.
    input_scales: [n_layers][4] scales of the (QKV, O, up, down) inputs.
    operand: see encoder_layer_fp8 (measurement only)."""
    layers = weights["layers"][:n_layers] if n_layers else weights["layers"]
    qw = qw if qw is not None else prepare_fp8({"layers": layers})
    h = _stacked_input(x, weights, operand)
    if h.shape[0] == 0:
        return np.zeros((0, h.shape[1]), dtype=np.float32)
    for i, lw in enumerate(layers):
        h = encoder_layer_fp8(h, lw, qw[i], input_scales[i], operand=operand)
    return layer_norm(h, weights["lnf_g"], weights["lnf_b"])


def calibrate(clips, weights, n_layers=None):
    """amax of every quantized linear map's input over a list of clips
    (waveforms), running the unquantized encoder: [n_layers][4]."""
    layers = weights["layers"][:n_layers] if n_layers else weights["layers"]
    amax = np.zeros((len(layers), 4), dtype=np.float64)
    for x in clips:
        h = _stacked_input(x, weights)
        if h.shape[0] == 0:
            continue
        for i, lw in enumerate(layers):
            rec = []
            h = encoder_layer_fp8(h, lw, None, None, record=rec)
            amax[i] = np.maximum(amax[i], rec)
    return amax


def scales_from_amax(amax):
    """Input scales amax / 448 (fp32); 1 where the amax is 0."""
    a = np.asarray(amax, dtype=np.float32)
    return np.where(a > 0, a / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
