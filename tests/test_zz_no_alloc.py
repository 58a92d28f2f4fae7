"""enc_forward_noalloc (the entry point that allocates nothing) against
enc_forward, through the C ABI, on MI355X.

Both run the same kernels; the no-allocation call takes its workspace, plan
arrays and split-K partial sums from the library's static scratch array
instead of context memory, so its embeddings must equal enc_forward's bit for
bit.  Two calls in a row, the second on a smaller batch, check that nothing
of the first call's scratch contents leaks into the second; a batch over the
scratch limit must fail before anything is enqueued.
"""

import sys

import numpy as np
import pytest

import oracle
from speech_audio_encoder_amd import workloads

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from speech_audio_encoder_amd import binding
    binding.load_library()
    say("enc_create (bf16, 32 layers)")
    enc = binding.Encoder(workloads.make_weights(32, bf16=True), dtype="bf16")
    yield torch, binding, enc
    enc.close()


def _out(torch, lengths):
    p_max = oracle.position_count(oracle.frame_count(int(max(lengths))))
    return torch.full((len(lengths), p_max, 1280), float("nan"), dtype=torch.bfloat16,
                      device="cuda")


def _both(torch, binding, enc, audio, lengths):
    dev = torch.from_numpy(np.ascontiguousarray(audio)).cuda()
    ref = enc.forward(dev, lengths, out=_out(torch, lengths))
    got = binding.enc_forward_noalloc(enc.ctx, dev, lengths, _out(torch, lengths))
    torch.cuda.synchronize()
    return got.float().cpu().numpy(), ref.float().cpu().numpy()


def test_noalloc_matches_enc_forward_two_calls(env):
    torch, binding, enc = env
    # first call: four clips, ragged tails, one too short for a position
    a1, l1 = workloads.custom_audio([480_000, 240_123, 16_000, 399], seed=201)
    say(f"call 1: lengths {list(map(int, l1))}")
    got1, ref1 = _both(torch, binding, enc, a1, l1)
    assert np.all(np.isfinite(ref1))
    np.testing.assert_array_equal(got1, ref1)
    # second call, smaller: the scratch still holds the first call's data
    a2, l2 = workloads.custom_audio([123_456, 400], seed=202)
    say(f"call 2: lengths {list(map(int, l2))}")
    got2, ref2 = _both(torch, binding, enc, a2, l2)
    np.testing.assert_array_equal(got2, ref2)
    for b, n in enumerate(l2):
        p = oracle.position_count(oracle.frame_count(int(n)))
        assert np.all(got2[b, p:] == 0.0)
    # and the no-allocation result is the oracle's to the embedding tolerance
    w = workloads.make_weights(32, bf16=True)
    ref = oracle.encode(a2[1, :400], w)
    err = float(np.abs(got2[1, :1] - ref).max())
    say(f"call 2 clip 1 vs oracle: {err:.3e} (max |ref| {np.abs(ref).max():.3f})")
    assert err <= 2e-2 * float(np.abs(ref).max())


def test_noalloc_windows_matches_enc_forward(env):
    torch, binding, enc = env
    a, l = workloads.custom_audio([700_000, 33_000], seed=203)
    enc.set_attention(200, 20)
    try:
        say("windows 200/20")
        got, ref = _both(torch, binding, enc, a, l)
    finally:
        enc.set_attention(None)
    np.testing.assert_array_equal(got, ref)


def test_noalloc_over_limit_fails_before_launch(env):
    torch, binding, enc = env
    lengths = [9_600_000]             # 7,500 positions: beyond the scratch limit
    need = binding.enc_workspace_bytes(32, lengths)
    assert need > (256 << 20) - (66 << 20)
    dev = torch.zeros((1, 9_600_000), dtype=torch.float32, device="cuda")
    out = _out(torch, lengths)
    code = binding.enc_forward_noalloc_raw(enc.ctx, dev.data_ptr(), lengths, out.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    assert code == binding.ENC_ERR_NOMEM, binding.enc_last_error()
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
