"""Build libqc.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m embedding_communication_codecs_amd.build

Flags that matter for bit-exact results: -ffp-contract=off (no fused
multiply-add in codec formulas); no fast-math, no flush-to-zero, and HIP's
correctly rounded fp32 division and square root are left on.  Packed fp32
instructions are switched off (-packed-fp32-ops): every fp32 operation is a
plain VALU op.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build", "qc")
LIB = os.path.join(PKG, "libqc.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]
SOURCES = ["k_encode.hip", "k_encode_codecs.hip", "k_encode_list.hip", "k_encode_list_codecs.hip", "k_fp8.hip", "k_decode.hip", "k_accumulate.hip", "k_vote.hip", "k_shared_sum.hip",
           "k_topk.hip", "qc_api.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx feature name and says so; harmless
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    """Compile every source and link libqc.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
