"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

    python gated_delta_rule_31_amd/build.py

(run as a file: the package itself refuses to import until the library exists)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = ["kda_api.hip", "kda_decode.hip", "kda_decode_multi.hip", "kda_decode_multi_seq.hip", "kda_prefill.hip",
           "kda_carry.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 ops (v_pk_*_f32) stay off: only scalar fp32 VALU is emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
