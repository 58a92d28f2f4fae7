"""Writes fp8_spread.txt: how far the FP8 oracle's own output moves under
two changes of rounding size upstream of its E4M3 decisions, as max and mean
|change| / max|output|:
  kind 0 -- its log-mel input moved by +-1e-4 (uniform, a tenth of the
            frontend's 1e-3 tolerance), a few trials;
  kind 1 -- the operands that the pages leave unquantized taken in bf16
            instead of float32: the input projection's stacked features and
            W_in, and the attention operands q, k, v (the ``operand`` map of
            oracle.fp8; the oracle itself keeps them in float32).

E4M3 codes are decisions (round to nearest on a grid with 2^-3 relative
steps): an input within rounding distance of a grid midpoint flips with any
upstream change, and the flip then propagates through every later layer.
The GPU's FP8 path and the oracle differ upstream by their frontend, by
their summation orders and by the GPU's bf16 operands, so they can agree
only up to this spread; the FP8 parity tests allow twice the largest value
found here at the same depth.

Calls only the oracle and the seeded input generators.  Run from the
repository root:  python tests/golden/fp8_spread.py  (about 5 minutes).
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import fp8  # noqa: E402
from oracle.encoder import layer_norm, linear  # noqa: E402
from oracle.frontend import logmel, stack_frames  # noqa: E402
from speech_audio_encoder_amd import workloads  # noqa: E402

AMAX = np.float32([5.0, 3.5, 5.0, 4.0])   # the parity tests' input amax per linear map


def spread(x, w, scales, qw, rng, trials):
    """[(kind, max move, mean move)] for one clip."""
    lm = logmel(x)
    outs = []
    for t in range(trials):
        noise = np.float32(1e-4) * rng.uniform(-1, 1, lm.shape) if t else 0.0
        h = linear(stack_frames((lm + noise).astype(np.float32)), w["w_in"], w["b_in"])
        for i, lw in enumerate(w["layers"]):
            h = fp8.encoder_layer_fp8(h, lw, qw[i], scales[i])
        outs.append((0, layer_norm(h, w["lnf_g"], w["lnf_b"])))
    outs.append((1, fp8.encode_fp8(x, w, scales, qw=qw, operand=fp8.round_bf16)))
    ref = outs[0][1]
    sc = np.abs(ref).max()
    return [(k, float(np.abs(o - ref).max() / sc), float(np.abs(o - ref).mean() / sc))
            for k, o in outs[1:]]


def main():
    rng = np.random.default_rng(1)
    rows = []
    w = workloads.make_weights(2, bf16=False, perturb=True)
    sc = np.tile(AMAX / np.float32(448), (2, 1))
    qw = fp8.prepare_fp8(w)
    audio, lengths = workloads.custom_audio([700_000, 33_000, 16_400, 400], seed=97)
    for b, n in enumerate(lengths):
        rows += [(2, m, a, k) for k, m, a in spread(audio[b, :n], w, sc, qw, rng, 6)]
    w = workloads.make_weights(32, bf16=True)
    sc = np.tile(AMAX / np.float32(448), (32, 1))
    qw = fp8.prepare_fp8(w)
    a, l = workloads.workload_audio("batch64")
    for b in (int(np.argmin(l)), 42):
        rows += [(32, m, mm, k) for k, m, mm in spread(a[b, :l[b]], w, sc, qw, rng, 4)]
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_spread.txt"), "w") as f:
        f.write("# layers max_move mean_move kind  (moves relative to max|output|; kind 0: "
                "log-mel +-1e-4, kind 1: bf16 operands), written by fp8_spread.py\n")
        for r in rows:
            f.write(f"{r[0]} {r[1]:.6f} {r[2]:.6f} {r[3]}\n")


if __name__ == "__main__":
    main()
