"""Plain, slow CPU oracle for the speech-encoder forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant generator with the HIP library under ``speech_audio_encoder_amd/``.

Source of the method: the page "Nemotron 3.5 Transcribe: From Recorded Speech
to Dataset Audits" (flozi.net), section "How audio and speakers reach the
language model": a 16 kHz mono waveform becomes 128 log-mel features (25 ms Hann
window, 512-point FFT, 10 ms hop); eight successive frames are stacked and
projected to width 1,280; 32 Transformer layers follow with ten heads, QK
normalisation, rotary position embeddings and a feed-forward expansion of four.

Precision: the frontend runs in float64 and is rounded to float32 once at the
end; the encoder runs in float32 (numpy BLAS), as the method specification for
this oracle fixes.

Every point the page leaves open is read one way, and the same reading is
stated next to the code that uses it (mel scale, window variant, norm type,
activation, RoPE pairing, block topology).
"""

from .frontend import (  # noqa: F401
    SAMPLE_RATE, WIN, HOP, NFFT, NBINS, NMELS, STACK, LOG_GUARD, MAX_SAMPLES,
    frame_count, position_count, hann_window, frame_signal, power_spectrum,
    hz_to_mel, mel_to_hz, mel_filterbank, logmel, logmel_batch, stack_frames,
)
from .encoder import (  # noqa: F401
    layer_norm, gelu, rope_tables, apply_rope, attention, encoder_layer,
    encode_from_logmel, encode, encode_windows, encode_batch, parameter_count,
)
from .fusion import (  # noqa: F401
    speaker_kernel, speaker_indicators, speaker_features, fuse_speakers, connector,
    encode_fused,
)
from . import fp8  # noqa: F401
from . import ctc  # noqa: F401
from . import align  # noqa: F401
