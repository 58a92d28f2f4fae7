"""The C-ABI library: it loads, exports every declared symbol, and its
host-only calls and argument checks behave as the header states (CPU only;
nothing here launches device work)."""

import ctypes
import os
import re

import numpy as np
import pytest

from speech_audio_encoder_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "speech_encoder.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|void|const char\*)\s+(enc_\w+)\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("enc_create", "enc_logmel", "enc_forward", "enc_destroy"):
        assert required in names
    assert sorted(binding.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


@pytest.mark.parametrize("n,f,p", [(0, 0, 0), (399, 0, 0), (400, 1, 1), (560, 2, 1),
                                   (16_000, 98, 13), (480_000, 2_998, 375),
                                   (57_600_000, 359_998, 45_000)])
def test_enc_shapes_closed_form(n, f, p):
    assert binding.enc_shapes([n]) == (f, p)


def test_enc_shapes_batch_uses_longest():
    assert binding.enc_shapes([400, 480_000, 16_000]) == (2_998, 375)


def test_argument_errors(lib):
    with pytest.raises(binding.EncoderError) as e:
        binding.enc_shapes([100, -1])
    assert e.value.code == binding.ENC_ERR_ARG
    with pytest.raises(binding.EncoderError) as e:
        binding.enc_shapes([57_600_001])
    assert e.value.code == binding.ENC_ERR_TOO_LONG
    assert "one hour" in binding.enc_last_error()
    f, p = ctypes.c_int64(), ctypes.c_int64()
    assert lib.enc_shapes(None, 1, ctypes.byref(f), ctypes.byref(p)) == binding.ENC_ERR_ARG
    arr = (ctypes.c_int64 * 1)(400)
    assert lib.enc_shapes(arr, 0, ctypes.byref(f), ctypes.byref(p)) == binding.ENC_ERR_ARG


def test_workspace_bytes_grows_with_positions():
    a = binding.enc_workspace_bytes(32, [480_000])
    b = binding.enc_workspace_bytes(32, [480_000, 480_000])
    assert 0 < a < b
    # at least the fp32 residual, bf16 activations, qkv and FFN buffers
    assert a >= 375 * (1280 * 4 + 1280 * 2 * 2 + 3840 * 2 + 5120 * 2)
    with pytest.raises(binding.EncoderError):
        binding.enc_workspace_bytes(0, [480_000])


def test_enc_create_rejects_bad_structs(lib):
    w = binding.EncWeights(abi_version=99, n_layers=1, dtype=binding.ENC_BF16)
    code, _ = binding.enc_create_raw(w)
    assert code == binding.ENC_ERR_ARG and "abi_version" in binding.enc_last_error()
    w = binding.EncWeights(abi_version=binding.ENC_ABI_VERSION, n_layers=0, dtype=binding.ENC_BF16)
    assert binding.enc_create_raw(w)[0] == binding.ENC_ERR_ARG
    w = binding.EncWeights(abi_version=binding.ENC_ABI_VERSION, n_layers=1, dtype=7)
    assert binding.enc_create_raw(w)[0] == binding.ENC_ERR_ARG
    w = binding.EncWeights(abi_version=binding.ENC_ABI_VERSION, n_layers=1, dtype=binding.ENC_F32)
    assert binding.enc_create_raw(w)[0] == binding.ENC_ERR_ARG   # NULL tensors
    assert lib.enc_create(None, None) == binding.ENC_ERR_ARG


def test_null_context_is_rejected(lib):
    arr = (ctypes.c_int64 * 1)(16000)
    assert lib.enc_forward(None, None, arr, 1, None, None) == binding.ENC_ERR_ARG
    assert lib.enc_logmel(None, None, arr, 1, None, None) == binding.ENC_ERR_ARG
    assert lib.enc_set_attention(None, binding.ENC_ATTN_WINDOWS, 500, 50) == binding.ENC_ERR_ARG
    assert lib.enc_set_connector(None, None) == binding.ENC_ERR_ARG
    assert lib.enc_set_precision(None, binding.ENC_PREC_BF16, None) == binding.ENC_ERR_ARG
    assert lib.enc_calibrate(None, None, arr, 1, None, None) == binding.ENC_ERR_ARG
    assert lib.enc_set_ctc(None, None) == binding.ENC_ERR_ARG
    assert lib.enc_forward_ctc(None, None, arr, 1, None, None) == binding.ENC_ERR_ARG
    assert lib.enc_forward_fused(None, None, arr, 1, None, None, None) == binding.ENC_ERR_ARG
    lib.enc_destroy(None)   # no-op


def test_packed_rows_closed_form():
    assert binding.packed_rows([0, 399, 400, 559, 560, 1680, 57_600_000]) == \
        0 + 0 + 1 + 1 + 1 + 2 + 45_000


def test_fp8_input_scales_host_call(lib):
    # amax / 448 in fp32, 1 for an all-zero input, errors for bad amax
    amax = np.array([[5.0, 0.0, 448.0, 1e-30]], np.float32)
    got = binding.scales_from_amax(amax)
    assert got.shape == amax.shape and got.dtype == np.float32
    assert got.tolist() == [[np.float32(5.0) / np.float32(448.0), 1.0, 1.0,
                             np.float32(1e-30) / np.float32(448.0)]]
    for bad in (-1.0, np.inf, np.nan):
        with pytest.raises(binding.EncoderError):
            binding.scales_from_amax(np.array([1.0, bad], np.float32))


def test_probe_peaks_argument_errors(lib):
    # checked on the host before anything reaches the device
    tf, gbs = ctypes.c_double(), ctypes.c_double()
    buf = ctypes.c_void_p(16)   # never dereferenced: every call below fails its checks
    assert lib.enc_probe_peaks(None, buf, 1 << 20, 1, None, ctypes.byref(tf),
                               ctypes.byref(gbs)) == binding.ENC_ERR_ARG
    assert lib.enc_probe_peaks(buf, buf, (1 << 20) + 8, 1, None, ctypes.byref(tf),
                               ctypes.byref(gbs)) == binding.ENC_ERR_ARG
    assert lib.enc_probe_peaks(buf, buf, 1 << 19, 1, None, ctypes.byref(tf),
                               ctypes.byref(gbs)) == binding.ENC_ERR_ARG
    assert lib.enc_probe_peaks(buf, buf, 1 << 20, 0, None, ctypes.byref(tf),
                               ctypes.byref(gbs)) == binding.ENC_ERR_ARG
    assert lib.enc_probe_peaks(buf, buf, 1 << 20, 1, None, None,
                               ctypes.byref(gbs)) == binding.ENC_ERR_ARG


def test_ctc_align_argument_errors(lib):
    # rejected on the host before any device work
    fr = (ctypes.c_int64 * 1)(10)
    nt = (ctypes.c_int64 * 1)(1)
    tk = (ctypes.c_int32 * 1)(3)
    assert lib.enc_ctc_align(None, None, 50, 50, fr, tk, nt, 1, None, None,
                             None) == binding.ENC_ERR_ARG
