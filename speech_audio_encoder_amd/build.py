"""Build libspeech_encoder.so (gfx950) in-tree with hipcc.

Usage: ``python -m speech_audio_encoder_amd.build`` (or ``build()``).  Each
source is compiled to an object under ``speech_audio_encoder_amd/_build`` in
parallel, then linked into ``speech_audio_encoder_amd/libspeech_encoder.so``.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libspeech_encoder.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["frontend.hip", "gemm.hip", "norm.hip", "attention.hip", "align.hip", "peak.hip",
           "runtime.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 instructions are switched off for every device compile.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-source additions.  attention.hip: MFMA results in VGPRs (its scores
# feed VALU work directly; the accumulators fit without AGPR staging).
EXTRA_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errors = [ln for ln in res.stderr.splitlines()
              if "packed-fp32-ops" not in ln]   # host-pass notice about the device flag
    return src, obj, res.returncode, "\n".join(errors)


def build(verbose=True, jobs=None):
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for src, obj, rc, err in results:
        if err.strip() and verbose:
            print(f"[build] {src}:\n{err}", file=sys.stderr)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"[build] wrote {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
