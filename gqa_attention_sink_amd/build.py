"""Build libsinkattn.so (gfx950) in-tree with hipcc.

    python -m gqa_attention_sink_amd.build        # or __graft_entry__.build()

Every HIP source is compiled with packed-FP32 instruction selection switched off.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libsinkattn.so")
SOURCES = ["api.hip", "prefill.hip", "decode.hip", "decode_stream.hip", "kv_append.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-ffp-contract=fast",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(os.path.dirname(PKG), "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the in-tree shared library; returns its path."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops" not in ln and "warning: argument unused" not in ln]
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
