"""Throughput of the speech-encoder forward pass on one MI355X.

One step = one ``enc_forward`` call over one batch of synthetic audio already
resident in HBM: log-mel frontend, 8-frame stack, input projection, 32
Transformer layers, final norm (bf16 operands, fp32 accumulation).  Prints one
JSON line with audio-seconds encoded per second, the achieved fraction of the
bf16 MFMA peak, the roofline of the dominant kernel (timed with HIP events on
the library's stream during the timed steps), the device's measured ceilings
(``measured_peaks``: a register-only bf16 MFMA loop and a 1 GiB device copy,
the library's probe kernels; ``--no-peak-probe`` skips them) and the CPU
oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                      [--attention CORE,CONTEXT] [--fused | --ctc [--align]]
                      [--precision bf16|fp8]
                      [--running-max-steps N]

--fused runs the encoder through speaker fusion and the 1280 -> 2688 connector
(synthetic speaker activity) instead of stopping at the embeddings.

--ctc runs the encoder and the CTC timestamp adapter (upsampling to the 40 ms
grid, two 16-head layers, 23,863-way projection, log-softmax) instead of
stopping at the embeddings; flops count the adapter at its real head width.
--align (implies --ctc) also force-aligns a synthetic token sequence per clip
onto the adapter's output in every step, and reports the alignment alone in
an "align" object.

--precision fp8 runs the four linear maps of every layer on E4M3 codes with
per-tensor scales (input scales from the library's calibration on the same
batch, untimed); GEMM flops are then priced at the fp8 MFMA peak.

--running-max-steps N (default 5) then times N steps of the same workload with
every layer's QK-norm gains tripled: the score bound then exceeds the fixed
softmax reference's range and the attention keeps a running maximum; the
line's "running_max" object gives that step time and its attention time.

--attention encodes each clip in windows of CORE positions with CONTEXT
positions of context on each side (500,50 are the serving windows, 375,0 the
30-second chunks); flops then count the windows' sequences, context included.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from speech_audio_encoder_amd import workloads  # noqa: E402

SAMPLE_RATE = 16000
D, FF, DIN, H, DH = 1280, 5120, 1024, 10, 128
LLM = 2688                     # language-model width (connector output)
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0

DESCRIPTIONS = {
    "tiny": "1 clip x 1.0 s tones, 2-layer encoder",
    "clip30": "1 clip x 30 s tones, 32-layer encoder",
    "batch64": "64 clips x U(5-30 s) tones (variable length, masked), 32-layer encoder",
    "long10m": "1 clip x 600 s segment mix, 32-layer encoder",
    "hour": "1 clip x 3600 s segment mix, 32-layer encoder",
}


def positions(n):
    f = 0 if n < 400 else 1 + (n - 400) // 160
    return (f + 7) // 8


def sequences(pos, core=0, context=0):
    """Lengths of the attention sequences the layers run on: whole clips, or
    each clip's windows (core positions plus context on each side)."""
    if core == 0:
        return list(pos)
    out = []
    for p in pos:
        for c0 in range(0, p, core):
            out.append(min(p, c0 + core + context) - max(0, c0 - context))
    return out


CTC_CLASSES, CTC_HEADS, CTC_DH, CTC_FFN = 23_863, 16, 80, 1280


def ctc_flops(clip_pos):
    """Algorithmic flops of the timestamp adapter on clips of P_b positions
    (2 P_b frames each): upsampling, two layers at head width 80, projection."""
    frames = [2 * p for p in clip_pos]
    r = sum(frames)
    layer = (2 * r * (3 * D * D + D * D + 2 * D * CTC_FFN)
             + sum(4 * f * f * CTC_DH * CTC_HEADS for f in frames))
    return 2 * sum(clip_pos) * D * 2 * D + 2 * layer + 2 * r * D * CTC_CLASSES


def gemm_flops_per_layer(rows):
    return 2 * rows * (3 * D * D + D * D + 2 * D * FF)


def attention_flops_per_layer(pos):
    return sum(4 * p * p * DH * H for p in pos)


def kernel_flops(name, rows, pos, clip_rows=None):
    """Algorithmic MFMA flops of one launch of a kernel class (rows: the
    layers' rows; clip_rows: the clips' positions, which the connector maps)."""
    return {
        "gemm_in": 2 * rows * D * DIN,
        "gemm_qkv": 2 * rows * 3 * D * D,
        "gemm_o": 2 * rows * D * D,
        "gemm_up": 2 * rows * D * FF,
        "gemm_down": 2 * rows * FF * D,
        "connector": 2 * (rows if clip_rows is None else clip_rows) * D * LLM,
        "attention": attention_flops_per_layer(pos),
    }.get(name)


def kernel_bytes(name, rows, lengths):
    """Algorithmic HBM bytes of one launch of the memory-bound kernel classes."""
    return {
        "frontend": 4 * int(sum(lengths)) + 2 * 128 * 8 * rows,   # audio in, bf16 stack out
        "layernorm": rows * D * (4 + 2),
        "qknorm_rope": rows * 2 * D * 2 * 2,                       # q and k read and written (bf16)
        "final_norm": rows * D * (4 + 2),
    }.get(name)


def class_rooflines(breakdown, rows, pos, lengths, clip_rows, fp8):
    """Each timed kernel class against its own bounds: algorithmic TFLOP/s
    over the MFMA peak (matrix-core classes) and algorithmic bytes / s over
    the HBM peak (row kernels; attention, which is both, gets both: q, k, v
    read and its output written once)."""
    out = {}
    for k, b in breakdown.items():
        if not b["launches"] or b["ms"] <= 0:
            continue
        t = b["ms"] / b["launches"] / 1000.0
        rec = {"us_per_launch": round(1e6 * t, 2)}
        fl = kernel_flops(k, rows, pos, clip_rows)
        if fl is not None:
            peak = PEAK_FP8_TFLOPS if fp8 and k in ("gemm_qkv", "gemm_o", "gemm_up",
                                                    "gemm_down") else PEAK_BF16_TFLOPS
            rec["tflops"] = round(fl / t / 1e12, 1)
            rec["frac_mfma"] = round(fl / t / 1e12 / peak, 4)
        by = kernel_bytes(k, rows, lengths)
        if k == "attention":
            by = 4 * rows * D * 2
        if by is not None:
            rec["tbps"] = round(by / t / 1e12, 3)
            rec["frac_hbm"] = round(by / t / 1e9 / PEAK_HBM_GBS, 4)
        out[k] = rec
    return out


def gemm_bytes(name, rows, fp8=False):
    """Algorithmic HBM bytes of one GEMM launch: A and W read once, C written
    once (bf16, E4M3 for the FP8 path's GELU output, or fp32 read+write for
    the residual epilogue)."""
    mnk = {"gemm_in": (D, DIN, 4), "gemm_qkv": (3 * D, D, 2), "gemm_o": (D, D, 8),
           "gemm_up": (FF, D, 1 if fp8 else 2), "gemm_down": (D, FF, 8)}.get(name)
    if mnk is None:
        return None
    n, k, c_bytes = mnk
    ab = 1 if fp8 and name != "gemm_in" else 2
    return rows * k * ab + n * k * ab + rows * n * c_bytes


def measured_traffic(workload, kernel):
    """HBM bytes per launch of a kernel class from the committed rocprofv3
    counter summary of this workload, if the kernel's sources are unchanged
    since the counters were taken (else None)."""
    from speech_audio_encoder_amd import prof_summary
    rec = prof_summary.read_traffic(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md"))
    if not rec or rec.get("workload") != workload:
        return None
    c = rec.get("classes", {}).get(kernel)
    if not c or c.get("sources_sha256") != prof_summary.source_hashes(kernel):
        return None
    return int(round(c["bytes_per_launch"]))


def stratified_order(lengths):
    """Clip indices in an order whose every prefix spreads evenly over the
    length range: the clips sorted by length, visited in bit-reversed rank
    order (van der Corput), so that a time-bounded sample is not biased to
    short or long clips."""
    ranked = np.argsort(lengths, kind="stable")
    n = len(ranked)
    bits = max(1, int(np.ceil(np.log2(max(n, 2)))))
    rev = sorted(range(1 << bits), key=lambda r: int(format(r, f"0{bits}b")[::-1], 2))
    return [int(ranked[r]) for r in rev if r < n]


def cpu_baseline(audio, lengths, weights, core=0, context=0, budget_s=12.0):
    """Time the oracle (as it stands) on whole clips until ~budget_s of CPU,
    the clips taken in an order spread evenly over the workload's lengths."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    order = stratified_order(lengths)
    done_samples, spent, clips = 0, 0.0, 0
    picked = []
    for b in order:
        n = int(lengths[b])
        t0 = time.perf_counter()
        if core:
            oracle.encode_windows(audio[b, :n], weights, core, context)
        else:
            oracle.encode(audio[b, :n], weights)
        spent += time.perf_counter() - t0
        done_samples += n
        clips += 1
        picked.append(n / SAMPLE_RATE)
        if spent >= budget_s:
            break
    secs = done_samples / SAMPLE_RATE
    all_s = np.asarray(lengths, dtype=np.float64) / SAMPLE_RATE
    return {"value": secs / spent, "unit": "audio-s/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{clips} of {len(lengths)} whole clip(s), spread evenly over the "
                      f"workload's lengths ({min(picked):.1f}-{max(picked):.1f} s, mean "
                      f"{np.mean(picked):.1f} s; workload mean {all_s.mean():.1f} s), "
                      f"{secs:.1f} audio-s, {len(weights['layers'])} layers, "
                      f"{spent:.1f} s wall"}


def score_log2_bound(lw):
    """Bound on |q.k| log2(e) / sqrt(w) from a layer's QK-norm parameters (a
    LayerNorm'd w-vector has norm <= sqrt(w)), with the library's 2^-6 margin;
    above 64 the attention keeps a running softmax maximum."""
    w = len(lw["q_g"])

    def norm_bound(g, b):
        g = np.asarray(g, dtype=np.float64)
        b = np.asarray(b, dtype=np.float64)
        return float(np.abs(g).max()) * np.sqrt(w) + float(np.linalg.norm(b))
    bound = norm_bound(lw["q_g"], lw["q_b"]) * norm_bound(lw["k_g"], lw["k_b"]) * (1 + 1 / 64)
    return bound * 1.4426950408889634 / np.sqrt(w)


def running_max_timing(weights, dtype, core, context, x, lengths, out, steps, stream):
    """Step time of the same workload with every layer's QK-norm gains tripled
    (same shapes and work; the attention takes its running-maximum softmax)."""
    import torch
    from speech_audio_encoder_amd import binding
    sharp = dict(weights)
    sharp["layers"] = [dict(lw, q_g=np.asarray(lw["q_g"]) * 3.0, k_g=np.asarray(lw["k_g"]) * 3.0)
                       for lw in weights["layers"]]
    bounds = [score_log2_bound(lw) for lw in sharp["layers"]]
    enc = binding.Encoder(sharp, dtype=dtype)
    if core:
        enc.set_attention(core, context)
    for _ in range(2):
        enc.forward(x, lengths, out=out)
    binding.enc_profile_kernel(enc.ctx, "attention")
    enc.forward(x, lengths, out=out)
    n_att, att_ms = binding.enc_profile_read(enc.ctx)
    binding.enc_profile_kernel(enc.ctx, -1)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        enc.forward(x, lengths, out=out)
    ev1.record(stream)
    torch.cuda.synchronize()
    enc.close()
    return {"qk_gain_scale": 3.0, "min_score_log2_bound": round(min(bounds), 2),
            "path": "running maximum" if min(bounds) > 64.0 else "fixed reference",
            "steps": steps, "ms_per_step": round(ev0.elapsed_time(ev1) / steps, 4),
            "attention_ms_per_step": round(att_ms, 4), "attention_launches": n_att}


def align_timing(enc, logprobs, frames, tokens, lengths, stream, reps=10):
    """The forced alignment alone (enc_ctc_align on the step's own adapter
    output), timed with HIP events on the library's stream."""
    import torch
    for _ in range(2):
        enc.ctc_align(logprobs, frames, tokens)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        enc.ctc_align(logprobs, frames, tokens)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    audio_s = sum(lengths) / SAMPLE_RATE
    return {"ms_per_call": round(ms, 4), "clips": len(frames), "frames": int(sum(frames)),
            "tokens": int(sum(len(t) for t in tokens)), "longest_clip_frames": int(max(frames)),
            "us_per_frame_of_longest_clip": round(1000.0 * ms / max(1, max(frames)), 3),
            "audio_s_per_s": round(audio_s / (ms / 1000.0), 1),
            "note": "one workgroup per clip; the frames of a clip are a sequential chain"}


def peak_probe(roof, nbytes=1 << 30, reps=5):
    """What the device sustains (the library's probe kernels: back-to-back bf16
    MFMAs on register operands, and a device copy of 1 GiB), with the dominant
    kernel's achieved rate as a fraction of it."""
    import torch
    from speech_audio_encoder_amd import binding
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    tflops, gbs = binding.enc_probe_peaks(dst, src, reps)
    del src, dst
    out = {"mfma_bf16_tflops": round(tflops, 1), "copy_gbs": round(gbs, 1),
           "copy_bytes": nbytes,
           "note": "register-only dense bf16 MFMA loop on every SIMD; device copy, "
                   "bytes read + written"}
    if roof.get("unit") == "TFLOP/s" and roof.get("peak") == PEAK_BF16_TFLOPS:
        out["dominant_frac_of_measured"] = round(roof["achieved"] / tflops, 4)
    elif roof.get("unit") == "GB/s":
        out["dominant_frac_of_measured"] = round(roof["achieved"] / gbs, 4)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batch64", choices=list(DESCRIPTIONS))
    ap.add_argument("--attention", default="full",
                    help="'full' or CORE,CONTEXT for windowed attention")
    ap.add_argument("--fused", action="store_true",
                    help="encoder + speaker fusion + connector (language-model input rows)")
    ap.add_argument("--align", action="store_true",
                    help="with --ctc: also force-align a synthetic token sequence per clip "
                         "(about six tokens per audio second) onto the adapter's output in "
                         "every step, and time the alignment alone")
    ap.add_argument("--ctc", action="store_true",
                    help="encoder + CTC timestamp adapter (log-probabilities on the 40 ms grid)")
    ap.add_argument("--precision", default="bf16", choices=["bf16", "fp8"],
                    help="linear maps of the layers in bf16 or FP8 (E4M3, per-tensor scales)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip timing every kernel class (one extra untimed step per "
                         "class); the roofline then takes the FFN-up GEMM")
    ap.add_argument("--running-max-steps", type=int, default=5,
                    help="after the timed steps, time this many steps of an encoder whose "
                         "QK-norm gains are tripled, so that attention keeps a running softmax "
                         "maximum (0: skip; plain bf16 forward only)")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip measuring the device's sustained MFMA rate and copy bandwidth")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times), "
                         "to scale HBM byte counters")
    args = ap.parse_args()
    core, context = 0, 0
    if args.attention != "full":
        core, context = (int(v) for v in args.attention.split(","))
        if core < 1 or context < 0:
            ap.error("--attention needs CORE >= 1 and CONTEXT >= 0")
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(splitting the encoder batch by clips across ranks is not implemented).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from speech_audio_encoder_amd import binding

    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": 5}), flush=True)
        return
    audio, lengths = workloads.workload_audio(args.workload)
    weights = workloads.workload_weights(args.workload)
    n_layers = len(weights["layers"])
    dtype = "bf16" if workloads.WORKLOADS[args.workload][3] else "f32"
    enc = binding.Encoder(weights, dtype=dtype)
    if core:
        enc.set_attention(core, context)
    x = torch.from_numpy(audio).cuda()
    lengths = [int(n) for n in lengths]
    pos = sequences([positions(n) for n in lengths], core, context)
    rows = sum(pos)
    _, p_max = binding.enc_shapes(lengths)
    stream = torch.cuda.current_stream()
    clip_pos = [positions(n) for n in lengths]
    fp8 = args.precision == "fp8"
    if fp8:
        amax = enc.calibrate(x, lengths)
        enc.set_precision("fp8", binding.scales_from_amax(amax))
    if args.align:
        args.ctc = True
    if args.ctc:
        enc.set_ctc(workloads.make_ctc_weights(bf16=True))
        out = torch.empty((2 * sum(clip_pos), enc.n_classes), dtype=torch.float32, device="cuda")
        align_frames = [2 * p for p in clip_pos]
        align_tokens = [workloads.alignment_case(0, min(f // 4, 1023), enc.n_classes, 500 + b)[1]
                        for b, f in enumerate(align_frames)]

        def step():
            enc.forward_ctc(x, lengths, out=out)
            if args.align:
                enc.ctc_align(out, align_frames, align_tokens)
    elif args.fused:
        cw = workloads.make_connector_weights(bf16=True)
        enc.set_connector(cw)
        acts = np.concatenate([workloads.speaker_activity(p, seed=400 + b)
                               for b, p in enumerate(clip_pos)])
        act_dev = torch.from_numpy(acts).cuda()
        out = torch.empty((sum(clip_pos), LLM), dtype=torch.bfloat16, device="cuda")

        def step():
            enc.forward_fused(x, lengths, act_dev, out=out)
    else:
        out = torch.empty((len(lengths), p_max, D), dtype=torch.bfloat16, device="cuda")

        def step():
            enc.forward(x, lengths, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    breakdown = {}
    if not args.no_breakdown:
        for kname in binding.KERNELS:
            binding.enc_profile_kernel(enc.ctx, kname)
            step()
            n, ms = binding.enc_profile_read(enc.ctx)
            breakdown[kname] = {"launches": n, "ms": round(ms, 4)}
        binding.enc_profile_kernel(enc.ctx, -1)
        torch.cuda.synchronize()

    # Dominant kernel: the slowest class per step that has a roofline model
    # (flops or bytes), from the breakdown; it is then bracketed with HIP
    # events on the library's stream during the timed steps.
    dom = "gemm_up"
    if breakdown:
        known = [k for k in breakdown if kernel_flops(k, 1, [1]) is not None
                 or kernel_bytes(k, 1, [1]) is not None]
        dom = max(known, key=lambda k: breakdown[k]["ms"])
    binding.enc_profile_kernel(enc.ctx, dom)

    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    n_dom, dom_ms = binding.enc_profile_read(enc.ctx)
    binding.enc_profile_kernel(enc.ctx, -1)

    ms_per_step = gpu_ms / args.steps
    audio_s = sum(lengths) / SAMPLE_RATE
    value = audio_s / (ms_per_step / 1000.0)
    total_flops = (n_layers * (gemm_flops_per_layer(rows) + attention_flops_per_layer(pos))
                   + 2 * rows * D * DIN)
    if args.fused:
        total_flops += 2 * sum(clip_pos) * D * LLM
    if args.ctc:
        total_flops += ctc_flops(clip_pos)
    if fp8:
        # layer GEMMs at the fp8 peak, attention and the bf16 products at the bf16 peak
        f8_flops = n_layers * gemm_flops_per_layer(rows)
        peak_time = (f8_flops / PEAK_FP8_TFLOPS + (total_flops - f8_flops) / PEAK_BF16_TFLOPS) / 1e12
        mfma_pct = 100.0 * peak_time / (ms_per_step / 1000.0)
    else:
        mfma_pct = 100.0 * total_flops / (ms_per_step / 1000.0) / (PEAK_BF16_TFLOPS * 1e12)

    avg_ms = dom_ms / max(n_dom, 1)
    fl = kernel_flops(dom, rows, pos, sum(clip_pos))
    traffic = measured_traffic(args.workload, dom)
    if fl is not None:
        achieved = fl / (avg_ms / 1000.0) / 1e12
        peak = PEAK_FP8_TFLOPS if fp8 and dom in ("gemm_qkv", "gemm_o", "gemm_up",
                                                  "gemm_down") else PEAK_BF16_TFLOPS
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic if not fp8 else None,
                "avg_launch_ms": round(avg_ms, 5), "launches": n_dom,
                "flops_per_launch": fl}
        ab = gemm_bytes(dom, rows, fp8)
        if ab is not None:
            roof["algorithmic_bytes_per_launch"] = ab
    else:
        by = kernel_bytes(dom, rows, lengths)
        achieved = by / (avg_ms / 1000.0) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic, "avg_launch_ms": round(avg_ms, 5), "launches": n_dom,
                "bytes_per_launch": by}
    if traffic is not None:
        roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, " \
                               "copy-calibrated)"

    result = {
        "metric": "audio-seconds encoded/sec (bf16 encoder fwd) + % MFMA peak, 1 MI355X",
        "value": round(value, 1),
        "unit": "audio-s/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "wall_ms_per_step": round(1000.0 * wall / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 layer GEMMs, bf16 attention" if fp8 else "bf16",
        "data": "synthetic",
        "mfma_pct_of_peak": round(mfma_pct, 2),
        "config": {"workload": f"{args.workload}: {DESCRIPTIONS[args.workload]}",
                   "clips": len(lengths), "audio_seconds": round(audio_s, 3),
                   "positions": sum(positions(n) for n in lengths), "layer_rows": rows,
                   "layers": n_layers,
                   "attention": "full" if not core else f"windows core={core} context={context}",
                   "precision": args.precision,
                   "output": "fused + connector rows [R, 2688]" if args.fused
                   else "CTC log-probabilities [2R, 23863] fp32 + forced alignment of "
                        "synthetic tokens" if args.align
                   else "CTC log-probabilities [2R, 23863] fp32" if args.ctc
                   else "embeddings [B, P_max, 1280]",
                   "algorithmic_tflop_per_step": round(total_flops / 1e12, 4)},
        "roofline": roof,
    }
    if breakdown:
        result["kernel_ms_per_step"] = breakdown
        result["class_rooflines"] = class_rooflines(breakdown, rows, pos, lengths,
                                                    sum(clip_pos), fp8)
    if args.align:
        result["align"] = align_timing(enc, out, align_frames, align_tokens, lengths, stream)
    enc.close()
    if args.running_max_steps > 0 and not (args.fused or args.ctc or fp8):
        result["running_max"] = running_max_timing(weights, dtype, core, context, x, lengths, out,
                                                   args.running_max_steps, stream)
    if not args.no_peak_probe:
        result["measured_peaks"] = peak_probe(roof)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(audio, lengths, weights, core, context)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
