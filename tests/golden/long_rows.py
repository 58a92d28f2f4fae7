"""Writes the stored 32-layer oracle rows of the two long recordings:

  * long10m_rows.npz -- 600 s segment mixture (seed 4), 7,500 positions,
    256 rows spread over the sequence (both ends, the 128-row tile edges
    near them, the middle, and seeded random rows);
  * hour_rows.npz    -- 3,600 s segment mixture (seed 5), 45,000 positions,
    64 rows (0, 1, 127, 128, 22,500, 44,871, 44,999 and seeded random rows).

Each file holds ``rows`` (int64 positions) and ``emb`` (float32 [len(rows),
1280]): the embeddings of those positions after all 32 layers and the final
LayerNorm, with full self-attention over the whole recording, from the bf16
weight draw.  Every earlier layer runs on all positions (keys and values need
them); only the last layer is limited to the stored rows (``rows=``), which
gives the same rows as the full computation.

The recordings and their sizes follow "Nemotron 3.5 Transcribe: From Recorded
Speech to Dataset Audits", section "How one hour fits into 65,536 positions"
(12.5 positions per second, 45,000 per hour) and section "Serving choices
that change the audit" (10-minute recordings).

Calls only the oracle and the seeded input generators.  Run from the
repository root, one workload per process if wanted:
    python tests/golden/long_rows.py long10m     (about 10 minutes on 8 cores)
    python tests/golden/long_rows.py hour        (about an hour on 8 cores)
"""

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from speech_audio_encoder_amd import workloads  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def stored_rows(name):
    """The positions whose oracle rows are stored for a workload."""
    if name == "long10m":
        p, n_rand = 7_500, 256
        fixed = [0, 1, 2, 63, 64, 127, 128, 129, 255, 256, 3_749, 3_750,
                 7_372, 7_423, 7_424, 7_487, 7_488, 7_498, 7_499]
    elif name == "hour":
        p, n_rand = 45_000, 64
        fixed = [0, 1, 127, 128, 22_500, 44_871, 44_999]
    else:
        raise ValueError(name)
    rng = np.random.default_rng(2024)
    rows = set(fixed)
    while len(rows) < n_rand:
        rows.add(int(rng.integers(0, p)))
    return np.array(sorted(rows), dtype=np.int64)


def path_for(name):
    return os.path.join(HERE, f"{name}_rows.npz")


def write(name):
    audio, lengths = workloads.workload_audio(name)
    w = workloads.make_weights(32, bf16=True)
    rows = stored_rows(name)
    t0 = time.perf_counter()
    print(f"[long_rows] {name}: {len(rows)} rows, 32 layers", flush=True)
    emb = oracle.encode(audio[0, :lengths[0]], w, rows=rows)
    assert emb.shape == (len(rows), workloads.D_MODEL) and np.all(np.isfinite(emb))
    np.savez(path_for(name), rows=rows, emb=emb.astype(np.float32))
    print(f"[long_rows] {name}: wrote {path_for(name)} in {time.perf_counter() - t0:.0f} s",
          flush=True)


if __name__ == "__main__":
    for arg in sys.argv[1:] or ["long10m", "hour"]:
        write(arg)
