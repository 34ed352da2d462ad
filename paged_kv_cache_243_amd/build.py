"""Build libpagedkv.so in place: every HIP source is compiled for gfx950 with
hipcc (in parallel, one object per source) and linked into one shared library
whose only runtime dependency is the HIP runtime.

    python -m paged_kv_cache_243_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libpagedkv.so")
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU instructions are kept out of every kernel.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{INCLUDE}", f"-I{CSRC}", "-Wno-unused-command-line-argument"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


# Per-source extra flags.  The prefill kernel never produces a NaN score
# (rows past seq_lens are zero-filled, masked scores are -inf), so its float
# max/min need no NaN quieting; its MFMAs keep results in VGPRs (the softmax
# reads every score, and AGPR results would each need a v_accvgpr_read, which
# contends with the MFMAs for the AGPR file).
EXTRA = {"prefill.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *EXTRA.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


# The benchmark's streaming-read ceiling kernel: its own small library beside
# bench.py, not part of libpagedkv.so.
CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_OUT = os.path.join(ROOT, "libbenchceiling.so")


def build_ceiling() -> str:
    tmp = CEILING_OUT + ".tmp"
    cmd = [HIPCC, *COMMON, "-shared", "-x", "hip", CEILING_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {CEILING_SRC}:\n{r.stderr}")
    os.replace(tmp, CEILING_OUT)
    return CEILING_OUT


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + 1)) as ex:
        ceiling = ex.submit(build_ceiling)
        objs = list(ex.map(_compile, srcs))
        ceiling.result()
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
