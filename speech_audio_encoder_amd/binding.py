"""ctypes binding of libspeech_encoder.so (the C ABI in include/speech_encoder.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  The
library is required: if it is missing this module raises instead of falling
back to anything else.

Function names follow the C calls: ``enc_create``, ``enc_logmel``,
``enc_forward``, ``enc_destroy``, ``enc_shapes``, ``enc_workspace_bytes``,
``enc_last_error``, ``enc_profile_kernel``, ``enc_profile_read``, ``enc_probe_peaks``,
``enc_ctc_align``.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspeech_encoder.so")

ENC_OK, ENC_ERR_ARG, ENC_ERR_TOO_LONG, ENC_ERR_NOMEM, ENC_ERR_HIP = 0, 1, 2, 3, 4
ENC_F32, ENC_BF16 = 0, 1
ENC_ABI_VERSION = 1
D_MODEL, N_MELS = 1280, 128

KERNELS = ["frontend", "gemm_in", "layernorm", "gemm_qkv", "qknorm_rope", "attention",
           "gemm_o", "gemm_up", "gemm_down", "final_norm", "speaker_fuse", "connector", "ctc",
           "ctc_out"]

EXPORTS = ["enc_create", "enc_logmel", "enc_forward", "enc_forward_noalloc", "enc_set_attention",
           "enc_set_connector",
           "enc_forward_fused", "enc_set_precision", "enc_calibrate", "enc_set_ctc",
           "enc_forward_ctc", "enc_fp8_input_scales", "enc_destroy", "enc_shapes",
           "enc_workspace_bytes", "enc_last_error", "enc_profile_kernel", "enc_profile_read",
           "enc_probe_peaks", "enc_ctc_align"]

ENC_PREC_BF16 = 0
ENC_PREC_FP8 = 1
E4M3_MAX = 448.0

ENC_ATTN_FULL = 0
ENC_ATTN_WINDOWS = 1

_LAYER_FIELDS = ["ln1_g", "ln1_b", "w_qkv", "b_qkv", "q_g", "q_b", "k_g", "k_b",
                 "w_o", "b_o", "ln2_g", "ln2_b", "w_up", "b_up", "w_down", "b_down"]


class EncLayerWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in _LAYER_FIELDS]


class EncWeights(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("w_in", ctypes.c_void_p), ("b_in", ctypes.c_void_p),
                ("layers", ctypes.POINTER(EncLayerWeights)),
                ("lnf_g", ctypes.c_void_p), ("lnf_b", ctypes.c_void_p)]


class EncConnectorWeights(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dim", ctypes.c_int32), ("speaker_scale", ctypes.c_float),
                ("spk_ln_g", ctypes.c_void_p), ("spk_ln_b", ctypes.c_void_p),
                ("w_conn", ctypes.c_void_p), ("b_conn", ctypes.c_void_p)]


class EncCtcWeights(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("n_classes", ctypes.c_int32),
                ("w_conv", ctypes.c_void_p), ("b_conv", ctypes.c_void_p),
                ("layers", ctypes.POINTER(EncLayerWeights)),
                ("lnf_g", ctypes.c_void_p), ("lnf_b", ctypes.c_void_p),
                ("w_out", ctypes.c_void_p), ("b_out", ctypes.c_void_p)]


class EncoderError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None


def load_library(path=LIB_PATH):
    """Open the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m speech_audio_encoder_amd.build`")
    lib = ctypes.CDLL(path)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.enc_create.argtypes = [ctypes.POINTER(EncWeights), ctypes.POINTER(ctypes.c_void_p)]
    lib.enc_logmel.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64p, ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_void_p]
    lib.enc_forward.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64p, ctypes.c_int32,
                                ctypes.c_void_p, ctypes.c_void_p]
    lib.enc_forward_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64p, ctypes.c_int32,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.enc_set_attention.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32]
    lib.enc_set_connector.argtypes = [ctypes.c_void_p, ctypes.POINTER(EncConnectorWeights)]
    lib.enc_forward_fused.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64p, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.enc_set_precision.argtypes = [ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.POINTER(ctypes.c_float)]
    lib.enc_calibrate.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64p, ctypes.c_int32,
                                  ctypes.POINTER(ctypes.c_float), ctypes.c_void_p]
    lib.enc_set_ctc.argtypes = [ctypes.c_void_p, ctypes.POINTER(EncCtcWeights)]
    lib.enc_forward_ctc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64p, ctypes.c_int32,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.enc_destroy.argtypes = [ctypes.c_void_p]
    lib.enc_destroy.restype = None
    lib.enc_shapes.argtypes = [i64p, ctypes.c_int32, i64p, i64p]
    lib.enc_workspace_bytes.argtypes = [ctypes.c_int32, i64p, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.enc_last_error.restype = ctypes.c_char_p
    lib.enc_last_error.argtypes = []
    lib.enc_fp8_input_scales.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_float)]
    lib.enc_profile_kernel.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    lib.enc_profile_read.argtypes = [ctypes.c_void_p, i64p, ctypes.POINTER(ctypes.c_double)]
    lib.enc_probe_peaks.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_int32, ctypes.c_void_p,
                                    ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double)]
    lib.enc_ctc_align.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                  i64p, ctypes.POINTER(ctypes.c_int32), i64p, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    for name in EXPORTS:
        if name not in ("enc_destroy", "enc_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def enc_last_error():
    return load_library().enc_last_error().decode()


def _check(code):
    if code != ENC_OK:
        raise EncoderError(code, enc_last_error())


def _lengths_array(lengths):
    arr = np.ascontiguousarray(np.asarray(lengths, dtype=np.int64).reshape(-1))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def enc_shapes(lengths):
    """(F_max, P_max) of a batch, computed by the library on the host."""
    arr, ptr = _lengths_array(lengths)
    f, p = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().enc_shapes(ptr, len(arr), ctypes.byref(f), ctypes.byref(p)))
    return f.value, p.value


def enc_workspace_bytes(n_layers, lengths):
    arr, ptr = _lengths_array(lengths)
    out = ctypes.c_size_t()
    _check(load_library().enc_workspace_bytes(n_layers, ptr, len(arr), ctypes.byref(out)))
    return out.value


def _stream_handle(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def enc_create(weights, dtype="bf16", device="cuda"):
    """Create a context from a weights dict (numpy or torch tensors).

    The tensors are put on the device in the requested element type for the
    duration of the call only: the library copies them into its own memory.
    Returns the context handle (an int).
    """
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    keep = []

    def dev(a):
        t = torch.as_tensor(np.asarray(a, dtype=np.float32)) if not torch.is_tensor(a) else a
        t = t.to(device=device, dtype=tdt).contiguous()
        keep.append(t)
        return ctypes.c_void_p(t.data_ptr())

    layers = (EncLayerWeights * len(weights["layers"]))()
    for i, lw in enumerate(weights["layers"]):
        for name in _LAYER_FIELDS:
            setattr(layers[i], name, dev(lw[name]))
    w = EncWeights(abi_version=ENC_ABI_VERSION, n_layers=len(weights["layers"]),
                   dtype=ENC_BF16 if dtype == "bf16" else ENC_F32, reserved=0,
                   w_in=dev(weights["w_in"]), b_in=dev(weights["b_in"]),
                   layers=layers, lnf_g=dev(weights["lnf_g"]), lnf_b=dev(weights["lnf_b"]))
    torch.cuda.synchronize()
    handle = ctypes.c_void_p()
    _check(load_library().enc_create(ctypes.byref(w), ctypes.byref(handle)))
    del keep
    return handle.value


def enc_create_raw(weights_struct):
    """enc_create on a caller-built EncWeights (for argument-check tests)."""
    handle = ctypes.c_void_p()
    code = load_library().enc_create(ctypes.byref(weights_struct), ctypes.byref(handle))
    return code, handle.value


def enc_destroy(ctx):
    load_library().enc_destroy(ctypes.c_void_p(ctx))


def enc_logmel(ctx, audio, lengths, out=None, stream=None):
    """Log-mel features: audio cuda fp32 [B, N_max] -> fp32 [B, F_max, 128]."""
    import torch
    arr, ptr = _lengths_array(lengths)
    f_max, _ = enc_shapes(arr)
    if out is None:
        out = torch.empty((len(arr), f_max, N_MELS), dtype=torch.float32, device=audio.device)
    _check(load_library().enc_logmel(ctypes.c_void_p(ctx), ctypes.c_void_p(audio.data_ptr()),
                                     ptr, len(arr), ctypes.c_void_p(out.data_ptr()),
                                     _stream_handle(stream)))
    return out


def enc_forward(ctx, audio, lengths, out=None, stream=None):
    """Embeddings: audio cuda fp32 [B, N_max] -> bf16 [B, P_max, 1280]."""
    import torch
    arr, ptr = _lengths_array(lengths)
    _, p_max = enc_shapes(arr)
    if out is None:
        out = torch.empty((len(arr), p_max, D_MODEL), dtype=torch.bfloat16, device=audio.device)
    _check(load_library().enc_forward(ctypes.c_void_p(ctx), ctypes.c_void_p(audio.data_ptr()),
                                      ptr, len(arr), ctypes.c_void_p(out.data_ptr()),
                                      _stream_handle(stream)))
    return out


def enc_forward_noalloc(ctx, audio, lengths, out, stream=None):
    """enc_forward through the entry point that allocates nothing; the caller
    passes the output ``out`` (bf16 [B, P_max, 1280])."""
    arr, ptr = _lengths_array(lengths)
    _check(load_library().enc_forward_noalloc(ctypes.c_void_p(ctx),
                                              ctypes.c_void_p(audio.data_ptr()), ptr, len(arr),
                                              ctypes.c_void_p(out.data_ptr()),
                                              _stream_handle(stream)))
    return out


def enc_forward_noalloc_raw(ctx, audio_ptr, lengths, out_ptr, stream_ptr=0):
    """enc_forward_noalloc with raw pointers; returns the status code (tests)."""
    arr, ptr = _lengths_array(lengths)
    return load_library().enc_forward_noalloc(ctypes.c_void_p(ctx), ctypes.c_void_p(audio_ptr),
                                              ptr, len(arr), ctypes.c_void_p(out_ptr),
                                              ctypes.c_void_p(stream_ptr))


def packed_rows(lengths):
    """Rows of the clip-packed layout: sum over clips of ceil(F_b / 8)."""
    total = 0
    for n in lengths:
        n = int(n)
        f = 0 if n < 400 else 1 + (n - 400) // 160
        total += (f + 7) // 8
    return total


def enc_set_connector(ctx, cw, dtype="bf16", device="cuda"):
    """Speaker-fusion and connector weights from a dict with spk_ln_g [8],
    spk_ln_b [8], w_conn [out_dim, 1280], b_conn [out_dim] and optionally
    speaker_scale (default 1)."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    keep = []

    def dev(a):
        t = torch.as_tensor(np.asarray(a, dtype=np.float32)) if not torch.is_tensor(a) else a
        t = t.to(device=device, dtype=tdt).contiguous()
        keep.append(t)
        return ctypes.c_void_p(t.data_ptr())

    w = EncConnectorWeights(abi_version=ENC_ABI_VERSION,
                            dtype=ENC_BF16 if dtype == "bf16" else ENC_F32,
                            out_dim=int(np.shape(cw["w_conn"])[0]),
                            speaker_scale=float(cw.get("speaker_scale", 1.0)),
                            spk_ln_g=dev(cw["spk_ln_g"]), spk_ln_b=dev(cw["spk_ln_b"]),
                            w_conn=dev(cw["w_conn"]), b_conn=dev(cw["b_conn"]))
    torch.cuda.synchronize()
    _check(load_library().enc_set_connector(ctypes.c_void_p(ctx), ctypes.byref(w)))
    del keep
    return w.out_dim


def enc_forward_fused(ctx, audio, lengths, activity, out_dim, out=None, stream=None):
    """Language-model input rows: audio cuda fp32 [B, N_max] and activity cuda
    fp32 [R, 8] (clips packed) -> bf16 [R, out_dim], R = packed_rows(lengths)."""
    import torch
    arr, ptr = _lengths_array(lengths)
    rows = packed_rows(arr)
    if tuple(activity.shape) != (rows, 8) or activity.dtype != torch.float32 \
            or not activity.is_contiguous():
        raise ValueError(f"activity must be contiguous float32 [{rows}, 8]")
    if out is None:
        out = torch.empty((rows, out_dim), dtype=torch.bfloat16, device=audio.device)
    _check(load_library().enc_forward_fused(
        ctypes.c_void_p(ctx), ctypes.c_void_p(audio.data_ptr()), ptr, len(arr),
        ctypes.c_void_p(activity.data_ptr()), ctypes.c_void_p(out.data_ptr()),
        _stream_handle(stream)))
    return out


def enc_set_precision(ctx, precision, input_scales=None):
    """ENC_PREC_BF16, or ENC_PREC_FP8 with input scales [n_layers, 4] (QKV, O,
    up, down inputs of each layer)."""
    ptr = None
    if input_scales is not None:
        arr = np.ascontiguousarray(input_scales, dtype=np.float32).reshape(-1)
        ptr = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    _check(load_library().enc_set_precision(ctypes.c_void_p(ctx), int(precision), ptr))


def enc_calibrate(ctx, audio, lengths, n_layers, stream=None):
    """amax [n_layers, 4] of the quantizable linear maps' inputs on one batch."""
    arr, ptr = _lengths_array(lengths)
    out = np.zeros(n_layers * 4, dtype=np.float32)
    _check(load_library().enc_calibrate(ctypes.c_void_p(ctx), ctypes.c_void_p(audio.data_ptr()),
                                        ptr, len(arr),
                                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)),
                                        _stream_handle(stream)))
    return out.reshape(n_layers, 4)


def scales_from_amax(amax):
    """Input scales from calibration amax values (the library's
    enc_fp8_input_scales), same shape, float32."""
    a = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty_like(a)
    fp = ctypes.POINTER(ctypes.c_float)
    _check(load_library().enc_fp8_input_scales(a.ctypes.data_as(fp), a.size,
                                               out.ctypes.data_as(fp)))
    return out


def enc_set_ctc(ctx, cw, dtype="bf16", device="cuda"):
    """Timestamp-adapter weights from a dict: w_conv [2, 1280, 1280] (tap,
    out, in), b_conv, layers (encoder-style dicts at head width 80), lnf_g,
    lnf_b, w_out [n_classes, 1280], b_out.  Returns n_classes."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    keep = []

    def dev(a):
        t = torch.as_tensor(np.asarray(a, dtype=np.float32)) if not torch.is_tensor(a) else a
        t = t.to(device=device, dtype=tdt).contiguous()
        keep.append(t)
        return ctypes.c_void_p(t.data_ptr())

    layers = (EncLayerWeights * len(cw["layers"]))()
    for i, lw in enumerate(cw["layers"]):
        for name in _LAYER_FIELDS:
            setattr(layers[i], name, dev(lw[name]))
    n_classes = int(np.shape(cw["w_out"])[0])
    w = EncCtcWeights(abi_version=ENC_ABI_VERSION, dtype=ENC_BF16 if dtype == "bf16" else ENC_F32,
                      n_layers=len(cw["layers"]), n_classes=n_classes,
                      w_conv=dev(cw["w_conv"]), b_conv=dev(cw["b_conv"]), layers=layers,
                      lnf_g=dev(cw["lnf_g"]), lnf_b=dev(cw["lnf_b"]), w_out=dev(cw["w_out"]),
                      b_out=dev(cw["b_out"]))
    torch.cuda.synchronize()
    _check(load_library().enc_set_ctc(ctypes.c_void_p(ctx), ctypes.byref(w)))
    del keep
    return n_classes


def enc_forward_ctc(ctx, audio, lengths, n_classes, out=None, stream=None):
    """CTC log-probabilities: audio cuda fp32 [B, N_max] -> fp32 [2 R, n_classes],
    clips packed in order (R = packed_rows(lengths))."""
    import torch
    arr, ptr = _lengths_array(lengths)
    rows = 2 * packed_rows(arr)
    if out is None:
        out = torch.empty((rows, n_classes), dtype=torch.float32, device=audio.device)
    _check(load_library().enc_forward_ctc(ctypes.c_void_p(ctx), ctypes.c_void_p(audio.data_ptr()),
                                          ptr, len(arr), ctypes.c_void_p(out.data_ptr()),
                                          _stream_handle(stream)))
    return out


def enc_forward_raw(ctx, audio_ptr, lengths, out_ptr, stream_ptr=0):
    """enc_forward with raw pointers; returns the status code (tests)."""
    arr, ptr = _lengths_array(lengths)
    return load_library().enc_forward(ctypes.c_void_p(ctx), ctypes.c_void_p(audio_ptr), ptr,
                                      len(arr), ctypes.c_void_p(out_ptr),
                                      ctypes.c_void_p(stream_ptr))


def enc_set_attention(ctx, mode, core=0, context=0):
    """Attention scope of later enc_forward calls: ENC_ATTN_FULL, or
    ENC_ATTN_WINDOWS with `core` positions per window plus `context` on each
    side."""
    _check(load_library().enc_set_attention(ctypes.c_void_p(ctx), int(mode), int(core),
                                            int(context)))


def enc_profile_kernel(ctx, name_or_id):
    kid = KERNELS.index(name_or_id) if isinstance(name_or_id, str) else int(name_or_id)
    _check(load_library().enc_profile_kernel(ctypes.c_void_p(ctx), kid))


def enc_profile_read(ctx):
    """(launches, total_ms) of the bracketed kernel since the last read."""
    n, ms = ctypes.c_int64(), ctypes.c_double()
    _check(load_library().enc_profile_read(ctypes.c_void_p(ctx), ctypes.byref(n),
                                           ctypes.byref(ms)))
    return n.value, ms.value


def enc_ctc_align(ctx, log_probs, frames, tokens_per_clip, n_classes, stream=None):
    """CTC forced alignment: log_probs cuda fp32 [sum frames, ld] (clip-packed,
    blank = n_classes - 1), frames [B], tokens_per_clip: B sequences of token
    ids -> (spans cuda int32 [sum L, 2], scores cuda fp32 [B])."""
    import torch
    fr, fr_ptr = _lengths_array(frames)
    nt = np.ascontiguousarray([len(t) for t in tokens_per_clip], dtype=np.int64)
    if len(nt) != len(fr):
        raise ValueError("one token sequence per clip")
    toks = np.ascontiguousarray(np.concatenate([np.asarray(t, dtype=np.int64).reshape(-1)
                                                for t in tokens_per_clip] or [np.zeros(0)]),
                                dtype=np.int32)
    n_tok = int(nt.sum())
    dev = log_probs.device
    spans = torch.empty((n_tok, 2), dtype=torch.int32, device=dev)
    scores = torch.empty(len(fr), dtype=torch.float32, device=dev)
    ld = log_probs.stride(0) if log_probs.dim() == 2 else n_classes
    _check(load_library().enc_ctc_align(
        ctypes.c_void_p(ctx), ctypes.c_void_p(log_probs.data_ptr()), int(ld), int(n_classes),
        fr_ptr, toks.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if n_tok else None,
        nt.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(fr),
        ctypes.c_void_p(spans.data_ptr()) if n_tok else None, ctypes.c_void_p(scores.data_ptr()),
        _stream_handle(stream)))
    return spans, scores


def enc_probe_peaks(dst, src, reps=5, stream=None):
    """(dense bf16 MFMA TFLOP/s, device-copy GB/s) measured on this device;
    dst and src are same-sized device tensors (>= 1 MiB, dst overwritten)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not (dst.is_cuda and src.is_cuda):
        raise ValueError("dst and src must be device tensors of the same size")
    tf, gbs = ctypes.c_double(), ctypes.c_double()
    _check(load_library().enc_probe_peaks(ctypes.c_void_p(dst.data_ptr()),
                                          ctypes.c_void_p(src.data_ptr()), nbytes, int(reps),
                                          _stream_handle(stream), ctypes.byref(tf),
                                          ctypes.byref(gbs)))
    return tf.value, gbs.value


class Encoder:
    """Owns one context; ``logmel`` and ``forward`` enqueue on torch's current stream."""

    def __init__(self, weights, dtype="bf16", device="cuda"):
        self.ctx = enc_create(weights, dtype=dtype, device=device)
        self.n_layers = len(weights["layers"])

    def logmel(self, audio, lengths, out=None):
        return enc_logmel(self.ctx, audio, lengths, out)

    def forward(self, audio, lengths, out=None):
        return enc_forward(self.ctx, audio, lengths, out)

    def set_connector(self, cw, dtype="bf16"):
        self.out_dim = enc_set_connector(self.ctx, cw, dtype=dtype)

    def forward_fused(self, audio, lengths, activity, out=None):
        return enc_forward_fused(self.ctx, audio, lengths, activity, self.out_dim, out)

    def set_ctc(self, cw, dtype="bf16"):
        self.n_classes = enc_set_ctc(self.ctx, cw, dtype=dtype)

    def forward_ctc(self, audio, lengths, out=None):
        return enc_forward_ctc(self.ctx, audio, lengths, self.n_classes, out)

    def ctc_align(self, log_probs, frames, tokens_per_clip, n_classes=None):
        return enc_ctc_align(self.ctx, log_probs, frames, tokens_per_clip,
                             n_classes if n_classes is not None else self.n_classes)

    def set_precision(self, precision, input_scales=None):
        """"bf16", or "fp8" with input scales [n_layers, 4]."""
        enc_set_precision(self.ctx, ENC_PREC_FP8 if precision == "fp8" else ENC_PREC_BF16,
                          input_scales)

    def calibrate(self, audio, lengths):
        return enc_calibrate(self.ctx, audio, lengths, self.n_layers)

    def set_attention(self, core=None, context=0):
        """Full-clip attention (core None) or windows of `core` positions with
        `context` positions of context on each side."""
        if core is None:
            enc_set_attention(self.ctx, ENC_ATTN_FULL, 0, 0)
        else:
            enc_set_attention(self.ctx, ENC_ATTN_WINDOWS, core, context)

    def close(self):
        if self.ctx:
            enc_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
