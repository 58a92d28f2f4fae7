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


def test_classify_fp8_layer_and_launch_counts():
    # the FP8 FFN up writes E4M3 codes (epilogue 4); it must not open a
    # residual run, or up and down would be taken for o and down
    fp8_layer = [k("layernorm_fp8_kernel"), gemm(0), k("qknorm_rope_kernel"),
                 k("attention_kernel<true>"), gemm(2), k("layernorm_fp8_kernel"), gemm(4),
                 gemm(2), gemm(2, True)]
    rows = [k("logmel_kernel<true>"), gemm(3)] + fp8_layer * 2
    got = [c for c, _ in prof_summary.classify(rows)]
    one = ["layernorm", "gemm_qkv", "qknorm_rope", "attention", "gemm_o", "layernorm",
           "gemm_up", "gemm_down", "gemm_down"]
    assert got == ["frontend", "gemm_in"] + one * 2
    per = prof_summary.class_launches(rows)
    assert {c: n for c, (_, n) in per.items()} == {
        "frontend": 1, "gemm_in": 1, "layernorm": 4, "gemm_qkv": 2, "qknorm_rope": 2,
        "attention": 2, "gemm_o": 2, "gemm_up": 2, "gemm_down": 2}
    assert len(per["gemm_down"][0]) == 4


def test_mfma_report_busy_share(tmp_path):
    # one GEMM dispatch, 1,024 SIMDs in 8 XCDs: GRBM_GUI_ACTIVE summed over the
    # XCDs is 8 x 1000 cycles, busy cycles summed over the SIMDs 512,000 ->
    # half the matrix-core cycles; 1e9 MOPS x 512 flops over 1 ms
    agent = tmp_path / "agent.csv"
    agent.write_text("Name,Simd_Count,Num_Xcc\ngfx950,1024,8\n")
    ctr = tmp_path / "ctr.csv"
    name = '"void enc::(anonymous namespace)::gemm_big_kernel<(enc::Epilogue)1, false>(int)"'
    lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"]
    for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 512000), ("GRBM_GUI_ACTIVE", 8000),
                 ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9)):
        lines.append(f"1,{name},{c},{v},0,1000000")
    ctr.write_text("\n".join(lines) + "\n")
    out = tmp_path / "m.md"
    prof_summary.mfma_report(str(ctr), str(agent), str(out), "cmd")
    row = [ln for ln in out.read_text().splitlines() if ln.startswith("| gemm_up")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "1" and cells[3] == "50.0%"
    assert cells[4] == "0.5120" and cells[5] == "512.0" and cells[6] == "20.5% bf16"


def _counter_csv(path, rows):
    """rows: (dispatch id, kernel name, counter, value, start, end)."""
    lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"]
    for d, n, c, v, t0, t1 in rows:
        lines.append(f'{d},"void enc::(anonymous namespace)::{n}(int)",{c},{v},{t0},{t1}')
    path.write_text("\n".join(lines) + "\n")


def test_lds_report_shares(tmp_path):
    # 256 CUs (1,024 SIMDs) in 8 XCDs; GRBM_GUI_ACTIVE summed over the XCDs is
    # 8 x 1000 cycles, so an average CU was active for 1000 of them: LDS active
    # 64,000 CU-cycles -> 25%, a quarter of those conflict cycles, MFMA busy
    # 102,400 SIMD-cycles -> 10%
    agent = tmp_path / "agent.csv"
    agent.write_text("Name,Simd_Count,Num_Xcc\ngfx950,1024,8\n")
    ctr = tmp_path / "ctr.csv"
    name = "attention_kernel<true, 128>"
    _counter_csv(ctr, [(1, name, c, v, 0, 2000) for c, v in (
        ("SQ_INSTS_LDS", 3e6), ("SQ_LDS_IDX_ACTIVE", 64000), ("SQ_LDS_BANK_CONFLICT", 16000),
        ("SQ_VALU_MFMA_BUSY_CYCLES", 102400), ("GRBM_GUI_ACTIVE", 8000))])
    out = tmp_path / "l.md"
    prof_summary.lds_report(str(ctr), str(agent), str(out), "cmd")
    row = [ln for ln in out.read_text().splitlines() if ln.startswith("| attention")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "1" and cells[2] == "2.0" and cells[3] == "3.00"
    assert cells[4] == "25.0%" and cells[5] == "25.0%" and cells[6] == "10.0%"


def test_counters_report_sums_per_launch_and_averages_latency(tmp_path):
    # two layers' LayerNorm launches: counters summed per launch (1 + 3 -> 2),
    # a derived latency averaged over the dispatches (100, 300 -> 200)
    ctr = tmp_path / "ctr.csv"
    rows = []
    for d, (w, lat) in enumerate([(1, 100), (3, 300)], start=1):
        rows.append((d, "layernorm_kernel", "SQ_WAIT_ANY", w, 0, 4000))
        rows.append((d, "layernorm_kernel", "VmemLatency", lat, 0, 4000))
    _counter_csv(ctr, rows)
    out = tmp_path / "c.md"
    prof_summary.counters_report(str(ctr), str(out), "cmd")
    text = out.read_text().splitlines()
    head = [ln for ln in text if ln.startswith("| class")][0]
    assert [c.strip() for c in head.strip("|").split("|")][3:] == ["SQ_WAIT_ANY", "VmemLatency"]
    row = [ln for ln in text if ln.startswith("| layernorm")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1] == "2" and cells[2] == "4.0" and cells[3] == "2" and cells[4] == "200"


def test_attention_key_runs_count_as_one_launch():
    # a key-split attention launch is the attention kernel followed by the
    # kernel that adds the runs' partial sums
    layer_split = [k("layernorm_kernel"), gemm(0), k("qknorm_rope_kernel"),
                   k("attention_kernel<true, 128>"), k("attention_combine_kernel<128>"), gemm(2),
                   k("layernorm_kernel"), gemm(1), gemm(2)]
    rows = [k("logmel_kernel<true>"), gemm(3)] + layer_split * 3
    per = prof_summary.class_launches(rows)
    assert per["attention"][1] == 3 and len(per["attention"][0]) == 6
    assert per["layernorm"][1] == 6
