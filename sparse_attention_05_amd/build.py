"""Build libdsa.so in-tree: every HIP source compiled by hipcc for gfx950, then linked.

    python -m sparse_attention_05_amd.build

Flags: -O3, gfx950 only; packed fp32 ops disabled (plain fp32 VALU code only).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdsa.so")
# the benchmark's measured-peak streams, kept out of the product library
PEAKS_LIB = os.path.join(HERE, "libdsa_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "quantize.hip", "index_rules.hip", "warmup.hip"]
# Per-source flags.  Inputs are NaN-free by contract (finite scales and bf16 values, no NaN
# fp8 codes), so fmaxf needs no NaN-quieting canonicalisation (the indexer's ReLU, the
# attention's running max).  Infinities are still honoured (masked logits are -inf).
EXTRA = {"indexer.hip": ["-fno-honor-nans"], "sparse_mla.hip": ["-fno-honor-nans"],
         "warmup.hip": ["-fno-honor-nans"]}
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH, "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall",
         "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB)
    if verbose:
        print("built", LIB, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
