"""Build libkq.so (gfx950) from csrc/ with hipcc.  Usage: python -m quant_weight_streaming_amd.build [--timeline]

--timeline builds libkq_timeline.so instead: the same sources with -DKQ_TIMELINE, whose chain kernel records
per-step device clock stamps (include/kq_timeline.h); it is for measurement only."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkq.so")
OUT_TIMELINE = os.path.join(HERE, "libkq_timeline.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["kq_gemv_q4k.hip", "kq_gemv_q5k.hip", "kq_gemv_q6k.hip", "kq_chain_bf16_lo.hip", "kq_chain_bf16_hi.hip",
           "kq_chain_f32.hip", "kq_chain_f32_wide.hip", "kq_chain_bf16_wide.hip", "kq_repack.hip", "kq_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-command-line-argument",
         # packed FP32 VALU forms stay out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, timeline: bool = False) -> str:
    bdir = BUILD + ("_timeline" if timeline else "")
    obj = os.path.join(bdir, os.path.basename(src) + ".o")
    flags = FLAGS + (["-DKQ_TIMELINE"] if timeline else [])
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-x", "hip", *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    out = OUT_TIMELINE if timeline else OUT
    os.makedirs(BUILD + ("_timeline" if timeline else ""), exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, timeline), SOURCES))
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True, timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
