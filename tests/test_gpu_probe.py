"""The device probes behind the bench line's measured peaks (MI355X)."""

import math

import pytest

pytestmark = pytest.mark.gpu


def test_probe_peaks_sane_and_copy_exact():
    import torch
    from speech_audio_encoder_amd import binding

    n = 64 << 20
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    tflops, gbs = binding.enc_probe_peaks(dst, src, reps=3)
    torch.cuda.synchronize()
    print(f"probe: {tflops:.1f} TFLOP/s bf16 MFMA, {gbs:.1f} GB/s copy of 64 MiB", flush=True)
    # the copy ran last: dst holds src bit for bit
    assert torch.equal(dst, src)
    assert math.isfinite(tflops) and math.isfinite(gbs)
    # within the published dense bf16 peak (2.5 PFLOP/s at 2.4 GHz) and well above
    # a tenth of it; a copy of 128 MiB moved (read + written) at a plausible rate
    assert 250.0 < tflops < 2600.0
    assert 100.0 < gbs < 20000.0
