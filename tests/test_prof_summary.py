"""Host logic of the rocprofv3 summaries: dispatches -> kernel classes."""

from speech_audio_encoder_amd import prof_summary


def k(name):
    return {"Kernel_Name": f"void enc::(anonymous namespace)::{name}(float const*, int)"}


def gemm(e, piece=False):
    kind = "gemm_piece_kernel" if piece else "gemm_big_kernel"
    extra = ", true" if piece else ""
    return k(f"{kind}<(enc::Epilogue){e}{extra}>")


def layer():
    return [k("layernorm_kernel"), gemm(0), gemm(0, True), k("qknorm_rope_kernel"),
            k("attention_kernel<true>"), gemm(2), k("layernorm_kernel"), gemm(1), gemm(2),
            gemm(2, True)]


def test_classify_plain_and_fused_steps():
    rows = [k("logmel_kernel<true>"), gemm(3)] + layer() + layer() + [k("final_norm_kernel")]
    rows += [k("logmel_kernel<true>"), k("gather_rows_kernel"), gemm(3)] + layer() + \
        [k("speaker_fuse_kernel"), gemm(0), gemm(0, True)]
    got = [c for c, _ in prof_summary.classify(rows)]
    one_layer = ["layernorm", "gemm_qkv", "gemm_qkv", "qknorm_rope", "attention", "gemm_o",
                 "layernorm", "gemm_up", "gemm_down", "gemm_down"]
    want = (["frontend", "gemm_in"] + one_layer * 2 + ["final_norm"]
            + ["frontend", "frontend", "gemm_in"] + one_layer
            + ["speaker_fuse", "connector", "connector"])
    assert got == want


def test_every_class_has_sources():
    for cls in prof_summary.CLASS_SOURCES:
        h = prof_summary.source_hashes(cls)
        assert h and all(len(v) == 64 for v in h.values())
