"""Summaries of rocprofv3 output for the encoder's kernels.

Reports, written as Markdown under ``profiles/``:

* ``kernels``: per-kernel calls / total / average duration from a
  ``--kernel-trace`` CSV (``<name>_kernel_trace.csv``);
* ``mfma``: matrix-core use per kernel class from one ``--pmc`` run of
  SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and the MFMA op counters
  (SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F8, add+mul ops / 512): busy share of
  all SIMDs' cycles while the GPU was active, and executed MFMA flops over
  the dispatch durations against the dtype's dense peak;
* ``l2``: L2 (TCC) hits and misses per launch of each class from one
  ``--pmc`` run of TCC_HIT_sum and TCC_MISS_sum;
* ``lds``: LDS instructions, LDS active share, bank-conflict cycles and MFMA
  busy share per class from one ``--pmc`` run of SQ_INSTS_LDS,
  SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT, SQ_VALU_MFMA_BUSY_CYCLES and
  GRBM_GUI_ACTIVE;
* ``counters``: any counters of one ``--pmc`` run per launch of each class
  (derived ``*Latency`` counters averaged over the dispatches);
* ``traffic``: HBM bytes per dispatch from two ``--pmc`` runs (FETCH_SIZE,
  WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
  for a plain device copy of known size (``bench.py --copy-calibration-mib``),
  grouped by the kernel classes the library times (``enc_profile_kernel``).
  The report ends with a JSON block that ``bench.py`` reads for the
  ``traffic`` field of its roofline; each class records the SHA-256 of the
  sources its kernels are built from, so a changed kernel reports no traffic.

Usage:
  python -m speech_audio_encoder_amd.prof_summary kernels TRACE_CSV OUT_MD "COMMAND"
  python -m speech_audio_encoder_amd.prof_summary mfma COUNTER_CSV AGENT_CSV OUT_MD "COMMAND" [SKIP]
  python -m speech_audio_encoder_amd.prof_summary l2 COUNTER_CSV OUT_MD "COMMAND"
  python -m speech_audio_encoder_amd.prof_summary lds COUNTER_CSV AGENT_CSV OUT_MD "COMMAND"
  python -m speech_audio_encoder_amd.prof_summary counters COUNTER_CSV OUT_MD "COMMAND"
  python -m speech_audio_encoder_amd.prof_summary traffic WORKLOAD FETCH_CSV WRITE_CSV \\
      COPY_FETCH_CSV COPY_WRITE_CSV COPY_MIB OUT_MD "COMMANDS"
"""

import collections
import csv
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# Kernel class -> sources its kernels come from.
CLASS_SOURCES = {
    "frontend": ["frontend.hip", "common.h", "kernels.h"],
    "gemm_in": ["gemm.hip", "common.h", "kernels.h"],
    "gemm_qkv": ["gemm.hip", "common.h", "kernels.h"],
    "gemm_o": ["gemm.hip", "common.h", "kernels.h"],
    "gemm_up": ["gemm.hip", "common.h", "kernels.h"],
    "gemm_down": ["gemm.hip", "common.h", "kernels.h"],
    "layernorm": ["norm.hip", "common.h", "kernels.h"],
    "qknorm_rope": ["norm.hip", "common.h", "kernels.h"],
    "attention": ["attention.hip", "common.h", "kernels.h"],
    "final_norm": ["norm.hip", "common.h", "kernels.h"],
    "speaker_fuse": ["norm.hip", "common.h", "kernels.h"],
    "connector": ["gemm.hip", "common.h", "kernels.h"],
}


def source_hashes(cls):
    out = {}
    for name in CLASS_SOURCES[cls]:
        with open(os.path.join(CSRC, name), "rb") as f:
            out[name] = hashlib.sha256(f.read()).hexdigest()
    return out


def short_name(name):
    n = re.sub(r"\(anonymous namespace\)::|enc::|^void ", "", name)
    n = re.sub(r"\(Epilogue\)", "E", n)
    return re.sub(r"\(.*", "", n) if "<" not in n else re.sub(r">\(.*", ">", n)


def epilogue_class(short):
    """Which GEMM a dispatch belongs to, from its epilogue (E0 bias->bf16:
    qkv, or the connector after the speaker fusion; E1 GELU and E4 GELU to
    E4M3: up; E2 residual: o and down alternate; E3 fp32: input)."""
    m = re.search(r"<E(\d)", short)
    return int(m.group(1)) if m else None


def classify(rows):
    """rows: dicts with Kernel_Name in dispatch order -> list of (class, row).
    A GEMM call is a contiguous run of dispatches with one epilogue (big-tile
    kernel, piece kernel, split-K reduce); residual-epilogue runs alternate
    between the attention output projection and the FFN contraction."""
    out = []
    e2_runs = 0
    prev_e2 = False
    after_fuse = False
    for r in rows:
        s = short_name(r["Kernel_Name"])
        cls, is_e2 = None, False
        if "logmel" in s or "gather_rows" in s:
            cls = "frontend"
            after_fuse = False
        elif s.startswith("speaker_fuse"):
            cls = "speaker_fuse"
            after_fuse = True
        elif s.startswith("layernorm"):
            cls = "layernorm"
        elif s.startswith("qknorm"):
            cls = "qknorm_rope"
        elif s.startswith("attention"):
            cls = "attention"
        elif s.startswith("final_norm"):
            cls = "final_norm"
        elif "gemm" in s or "splitk" in s:
            e = epilogue_class(s)
            if e == 0:
                cls = "connector" if after_fuse else "gemm_qkv"
            elif e in (1, 4):
                cls = "gemm_up"
            elif e == 3:
                cls = "gemm_in"
            else:
                is_e2 = True
                if not prev_e2:
                    e2_runs += 1
                cls = "gemm_o" if e2_runs % 2 == 1 else "gemm_down"
        prev_e2 = is_e2
        out.append((cls, r))
    return out


SINGLE_KERNEL = ("layernorm", "final_norm", "qknorm_rope", "attention", "speaker_fuse")


def _dur_us(r):
    return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0


def class_launches(rows):
    """rows in dispatch order -> {class: (its dispatches, launches)}: a
    launch is a run of consecutive dispatches of one class (a GEMM's big-tile
    kernel, tail pieces and split-K reduce), or each dispatch of a class whose
    launcher issues one kernel."""
    per = collections.OrderedDict()
    prev = None
    for cls, r in classify(rows):
        if cls is None:
            prev = None
            continue
        e = per.setdefault(cls, [[], 0])
        e[0].append(r)
        # the kernel that adds key runs' partial sums belongs to the
        # attention launch before it
        cont = cls == prev and short_name(r["Kernel_Name"]).startswith("attention_combine")
        if cls != prev or (cls in SINGLE_KERNEL and not cont):
            e[1] += 1
        prev = cls
    return per


def kernels_report(trace_csv, out_md, command):
    rows = list(csv.DictReader(open(trace_csv)))
    agg = collections.OrderedDict()
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        agg.setdefault(short_name(r["Kernel_Name"]), []).append(d)
    tot = sum(sum(v) for v in agg.values())
    lines = ["# Kernel durations: " + os.path.basename(out_md)[:-3], "",
             "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | total ms | avg us | share |", "|---|---:|---:|---:|---:|"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / 1000:.3f} | {sum(v) / len(v):.2f} | "
                     f"{100 * sum(v) / tot:.1f}% |")
    # Per kernel class (the units bench.py times with HIP events): a class
    # launch is one call of the library's launcher, e.g. a GEMM's big-tile
    # kernel plus its tail pieces and split-K reduce.
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    per = collections.OrderedDict(
        (cls, [sum(_dur_us(r) for r in rs), n]) for cls, (rs, n) in class_launches(rows).items())
    lines += ["", "Per kernel class (one launch = one call of the library's launcher; "
              "dispatch durations summed):", "",
              "| class | launches | avg us per launch |", "|---|---:|---:|"]
    for cls, (t, n) in per.items():
        lines.append(f"| {cls} | {n} | {t / max(n, 1):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


# Dense MFMA peaks of one MI355X (TFLOP/s), per operand type.
MFMA_PEAK = {"bf16": 2500.0, "fp8": 5000.0}
MOPS = {"bf16": "SQ_INSTS_VALU_MFMA_MOPS_BF16", "fp8": "SQ_INSTS_VALU_MFMA_MOPS_F8"}


def mfma_report(counter_csv, agent_csv, out_md, command, skip=0):
    """Per kernel class: MFMA busy share and executed MFMA throughput.

    SQ_VALU_MFMA_BUSY_CYCLES counts per SIMD and GRBM_GUI_ACTIVE per XCD;
    rocprofv3 sums each over its instances, so the busy share is
    busy / (gui_active / n_xcd * n_simd).  The op counters count add and mul
    operations / 512, so executed flops = ops * 512 (padding rows and masked
    attention tiles included: the MFMAs a kernel issues, not the algorithm's
    count).  skip: encoder passes (each opens with its log-mel dispatch) to
    leave out at the start, e.g. an untimed calibration pass."""
    agent = [r for r in csv.DictReader(open(agent_csv)) if int(r.get("Simd_Count") or 0) > 0][0]
    n_simd, n_xcd = int(agent["Simd_Count"]), int(agent["Num_Xcc"])
    disp = collections.OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        d = disp.setdefault(int(r["Dispatch_Id"]), dict(r))
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    rows = sorted(disp.values(), key=lambda r: int(r["Start_Timestamp"]))
    if skip:
        starts = [i for i, r in enumerate(rows) if "logmel" in short_name(r["Kernel_Name"])]
        rows = rows[starts[skip]:] if len(starts) > skip else []
    types = [t for t in MOPS if MOPS[t] in rows[0]] if rows else []
    lines = ["# MFMA use per kernel class: " + os.path.basename(out_md)[:-3], "",
             "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             f"Agent: {agent.get('Name', '')}, {n_simd} SIMDs in {n_xcd} XCDs.  MFMA busy = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs), summed over the "
             "class's dispatches; executed TFLOP = MFMA ops x 512 from the op counters; "
             "TFLOP/s = executed flops / summed dispatch durations (counter collection "
             "serialises dispatches, so short kernels read slightly low).", "",
             "| class | launches | avg us | MFMA busy | " +
             " | ".join(f"{t} TFLOP/launch" for t in types) + " | TFLOP/s | % of peak |",
             "|---|---:|---:|---:|" + "---:|" * len(types) + "---:|---:|"]
    for cls, (rs, n) in class_launches(rows).items():
        busy = sum(r.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for r in rs)
        gui = sum(r.get("GRBM_GUI_ACTIVE", 0.0) for r in rs)
        t_s = sum(_dur_us(r) for r in rs) / 1e6
        fl = {t: sum(r.get(MOPS[t], 0.0) for r in rs) * 512 for t in types}
        share = 100.0 * busy / (gui / n_xcd * n_simd) if gui else 0.0
        rate = sum(fl.values()) / t_s / 1e12 if t_s else 0.0
        # peak of the dominant operand type
        dom = max(types, key=lambda t: fl[t]) if types and sum(fl.values()) else None
        pct = f"{100 * rate / MFMA_PEAK[dom]:.1f}% {dom}" if dom else "-"
        lines.append(f"| {cls} | {n} | {1e6 * t_s / max(n, 1):.1f} | {share:.1f}% | " +
                     " | ".join(f"{fl[t] / max(n, 1) / 1e12:.4f}" for t in types) +
                     f" | {rate:.1f} | {pct} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter(path, counter):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    key = "Dispatch_Id" if rows and "Dispatch_Id" in rows[0] else None
    if key:
        rows.sort(key=lambda r: int(r[key]))
    return rows


def traffic_report(workload, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_mib,
                   out_md, commands):
    copy_bytes = copy_mib * (1 << 20)

    def calib(path, counter):
        vals = [float(r["Counter_Value"]) for r in _counter(path, counter)
                if "copy" in r["Kernel_Name"].lower()]
        vals = [v for v in vals if v > 0.25 * copy_bytes / 1024]   # the 1-GiB copies
        med = sorted(vals)[len(vals) // 2]
        return copy_bytes / (med * 1024.0), med

    f_fac, f_med = calib(copy_fetch_csv, "FETCH_SIZE")
    w_fac, w_med = calib(copy_write_csv, "WRITE_SIZE")
    per_class = {}
    for counter, path, fac in (("FETCH_SIZE", fetch_csv, f_fac), ("WRITE_SIZE", write_csv, w_fac)):
        rows = _counter(path, counter)
        for cls, r in classify(rows):
            if cls is None:
                continue
            d = per_class.setdefault(cls, {"FETCH_SIZE": [], "WRITE_SIZE": [], "kernels": set()})
            d[counter].append(float(r["Counter_Value"]) * 1024.0 * fac)
            d["kernels"].add(short_name(r["Kernel_Name"]))
    calls = {"frontend": 1, "gemm_in": 1, "final_norm": 1, "speaker_fuse": 1, "connector": 1,
             "layernorm": 2}
    record = {"workload": workload, "fetch_factor": f_fac, "write_factor": w_fac, "classes": {}}
    lines = ["# HBM traffic per launch: " + workload, "",
             "Commands (from the repository root, on one MI355X; each counter in a run",
             "of its own):", "", "```", commands, "```", "",
             f"Calibration: a plain {copy_mib} MiB device copy reads {f_med:.0f} KiB on "
             f"FETCH_SIZE (factor {f_fac:.3f}) and {w_med:.0f} KiB on WRITE_SIZE "
             f"(factor {w_fac:.3f}); counters below are scaled by those factors.", "",
             "Per launch of a kernel class = the sum over its dispatches in one step divided "
             "by the class's launches per step (layers, or 2 x layers for LayerNorm).", "",
             "| class | kernels | fetch MB/launch | write MB/launch | total MB/launch |",
             "|---|---|---:|---:|---:|"]
    # one log-mel dispatch per step
    n_steps = sum(1 for r in _counter(fetch_csv, "FETCH_SIZE")
                  if "logmel" in short_name(r["Kernel_Name"])) or 1
    for cls in CLASS_SOURCES:
        if cls not in per_class:
            continue
        d = per_class[cls]
        launches_per_step = calls.get(cls)
        if launches_per_step is None:
            # per-layer classes: dispatches of the class / kernels per call
            launches_per_step = max(1, len(d["FETCH_SIZE"]) // n_steps //
                                    max(1, len(d["kernels"])))
        elif cls == "layernorm":
            launches_per_step = len(d["FETCH_SIZE"]) // n_steps
        n_launch = n_steps * launches_per_step
        fb = sum(d["FETCH_SIZE"]) / n_launch
        wb = sum(d["WRITE_SIZE"]) / n_launch
        lines.append(f"| {cls} | {', '.join(f'`{k}`' for k in sorted(d['kernels']))} | "
                     f"{fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} |")
        record["classes"][cls] = {"fetch_bytes": fb, "write_bytes": wb,
                                  "bytes_per_launch": fb + wb, "sources_sha256": source_hashes(cls)}
    lines += ["", "Machine-readable record (read by bench.py):", "", "```json",
              json.dumps(record, indent=1, sort_keys=True), "```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def l2_report(counter_csv, out_md, command):
    """Per kernel class: L2 (TCC) hits and misses per launch from one --pmc
    run of TCC_HIT_sum and TCC_MISS_sum, and the hit rate.  A miss goes to
    the data fabric (the memory-side Infinity Cache, then HBM), so misses
    bound the fetch traffic of a class from above of what HBM itself serves."""
    disp = collections.OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        d = disp.setdefault(int(r["Dispatch_Id"]), dict(r))
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    rows = sorted(disp.values(), key=lambda r: int(r["Start_Timestamp"]))
    lines = ["# L2 hits and misses per kernel class: " + os.path.basename(out_md)[:-3], "",
             "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             "TCC_HIT_sum and TCC_MISS_sum summed over the class's dispatches (all eight XCDs' "
             "L2s), per launch of the class.", "",
             "| class | launches | L2 hits / launch (M) | L2 misses / launch (M) | hit rate |",
             "|---|---:|---:|---:|---:|"]
    for cls, (rs, n) in class_launches(rows).items():
        hit = sum(r.get("TCC_HIT_sum", 0.0) for r in rs)
        miss = sum(r.get("TCC_MISS_sum", 0.0) for r in rs)
        rate = 100.0 * hit / (hit + miss) if hit + miss else 0.0
        lines.append(f"| {cls} | {n} | {hit / max(n, 1) / 1e6:.2f} | {miss / max(n, 1) / 1e6:.2f} | "
                     f"{rate:.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def lds_report(counter_csv, agent_csv, out_md, command):
    """Per kernel class: LDS and matrix-core activity from one --pmc run of
    SQ_INSTS_LDS, SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT,
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE.  The LDS counters are summed
    over the CUs, the MFMA counter over the SIMDs and GRBM_GUI_ACTIVE over the
    XCDs, so a share is the counter / (GRBM_GUI_ACTIVE / XCDs x units)."""
    agent = [r for r in csv.DictReader(open(agent_csv)) if int(r.get("Simd_Count") or 0) > 0][0]
    n_simd, n_xcd = int(agent["Simd_Count"]), int(agent["Num_Xcc"])
    n_cu = n_simd // 4
    disp = collections.OrderedDict()
    for r in csv.DictReader(open(counter_csv)):
        d = disp.setdefault(int(r["Dispatch_Id"]), dict(r))
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    rows = sorted(disp.values(), key=lambda r: int(r["Start_Timestamp"]))
    lines = ["# LDS and MFMA activity per kernel class: " + os.path.basename(out_md)[:-3], "",
             "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             f"Agent: {agent.get('Name', '')}, {n_cu} CUs ({n_simd} SIMDs) in {n_xcd} XCDs.  "
             "LDS active = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / XCDs x CUs): the share of "
             "the class's time the LDS of an average CU spends on indexed reads and writes; "
             "conflict = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; MFMA busy as in the MFMA "
             "report.", "",
             "| class | launches | avg us | LDS instr / launch (M) | LDS active | "
             "bank-conflict cycles | MFMA busy |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    for cls, (rs, n) in class_launches(rows).items():
        gui = sum(r.get("GRBM_GUI_ACTIVE", 0.0) for r in rs)
        act = sum(r.get("SQ_LDS_IDX_ACTIVE", 0.0) for r in rs)
        conf = sum(r.get("SQ_LDS_BANK_CONFLICT", 0.0) for r in rs)
        ins = sum(r.get("SQ_INSTS_LDS", 0.0) for r in rs)
        busy = sum(r.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for r in rs)
        t_us = sum(_dur_us(r) for r in rs)
        per_unit = gui / n_xcd if gui else 0.0
        lds = 100.0 * act / (per_unit * n_cu) if per_unit else 0.0
        mf = 100.0 * busy / (per_unit * n_simd) if per_unit else 0.0
        cf = 100.0 * conf / act if act else 0.0
        lines.append(f"| {cls} | {n} | {t_us / max(n, 1):.1f} | {ins / max(n, 1) / 1e6:.2f} | "
                     f"{lds:.1f}% | {cf:.1f}% | {mf:.1f}% |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def counters_report(counter_csv, out_md, command):
    """Per kernel class: every counter of one --pmc run per launch (summed
    over the class's dispatches), except derived latencies (names ending in
    "Latency", in cycles), which are averaged over the dispatches."""
    disp = collections.OrderedDict()
    names = []
    for r in csv.DictReader(open(counter_csv)):
        d = disp.setdefault(int(r["Dispatch_Id"]), dict(r))
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        if r["Counter_Name"] not in names:
            names.append(r["Counter_Name"])
    rows = sorted(disp.values(), key=lambda r: int(r["Start_Timestamp"]))
    lines = ["# Counters per kernel class: " + os.path.basename(out_md)[:-3], "",
             "Command (from the repository root, on one MI355X):", "", "```", command, "```", "",
             "Per launch of the class (sum over its dispatches); `*Latency`: mean over the "
             "dispatches, in cycles.", "",
             "| class | launches | avg us | " + " | ".join(names) + " |",
             "|---|---:|---:|" + "---:|" * len(names)]
    for cls, (rs, n) in class_launches(rows).items():
        vals = []
        for k in names:
            v = [r.get(k, 0.0) for r in rs]
            vals.append(sum(v) / len(v) if k.endswith("Latency") else sum(v) / max(n, 1))
        t_us = sum(_dur_us(r) for r in rs) / max(n, 1)
        lines.append(f"| {cls} | {n} | {t_us:.1f} | " + " | ".join(f"{v:.4g}" for v in vals) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def read_traffic(md_path):
    """The JSON record at the end of a traffic report, or None."""
    try:
        text = open(md_path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    return json.loads(m.group(1)) if m else None


if __name__ == "__main__":
    if sys.argv[1] == "kernels":
        kernels_report(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "mfma":
        mfma_report(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5],
                    int(sys.argv[6]) if len(sys.argv) > 6 else 0)
    elif sys.argv[1] == "l2":
        l2_report(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "counters":
        counters_report(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "lds":
        lds_report(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif sys.argv[1] == "traffic":
        traffic_report(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6],
                       int(sys.argv[7]), sys.argv[8], sys.argv[9])
    else:
        sys.exit(__doc__)
