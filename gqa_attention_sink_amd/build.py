"""Build libsinkattn.so (gfx950) in-tree with hipcc.

    python -m gqa_attention_sink_amd.build        # or __graft_entry__.build()
    python -m gqa_attention_sink_amd.build host-sanitized

Every HIP source is compiled with packed-FP32 instruction selection switched off.  The
C ABI layer (api.cpp) is plain host C++; ``build_host_sanitized()`` compiles it with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer against a stub of the launch
layer (no device code), for the host-side validation and planning tests.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
LIB = os.path.join(PKG, "libsinkattn.so")
HOST_SAN_LIB = os.path.join(PKG, "libsinkattn_host_asan.so")
PEAK_LIB = os.path.join(PKG, "libsinkattn_peak.so")   # achievable-peak probes (bench only)
HOST_SOURCES = ["api.cpp"]
HIP_SOURCES = ["runtime.hip", "noalloc.hip", "prefill.hip", "decode.hip", "decode_stream.hip", "kv_append.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_INCLUDE = "/opt/rocm/include"

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
    "-I", INCLUDE,
    "-I", ROCM_INCLUDE,
    "-D__HIP_PLATFORM_AMD__",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"{cmd[0]} failed with exit code {res.returncode}")
    return res


def build(verbose: bool = False) -> str:
    """Compile every source into the in-tree shared library; returns its path."""
    host = [os.path.join(CSRC, s) for s in HOST_SOURCES]
    hip = [os.path.join(CSRC, s) for s in HIP_SOURCES]
    tmp = LIB + ".tmp"
    res = _run([HIPCC, *FLAGS, "-x", "c++", *host, "-x", "hip", *hip, "-o", tmp], verbose)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops" not in ln and "warning: argument unused" not in ln]
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, LIB)
    tmp = PEAK_LIB + ".tmp"
    _run([HIPCC, *FLAGS, "-x", "hip", os.path.join(CSRC, "peak_probe.hip"), "-o", tmp], verbose)
    os.replace(tmp, PEAK_LIB)
    return LIB


def build_host_sanitized(verbose: bool = False) -> str:
    """Host-only build of the C ABI layer with ASan + UBSan (g++, no device code): the
    launch layer is a stub that reports no device, so every validation and planning
    path runs as in the library.  Load it with the ASan runtime preloaded."""
    cxx = os.environ.get("CXX", "g++")
    srcs = [os.path.join(CSRC, s) for s in HOST_SOURCES + ["host_stub.cpp"]]
    tmp = HOST_SAN_LIB + ".tmp"
    _run([cxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-I", INCLUDE, "-I", ROCM_INCLUDE,
          "-D__HIP_PLATFORM_AMD__", *srcs, "-o", tmp], verbose)
    os.replace(tmp, HOST_SAN_LIB)
    return HOST_SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "host-sanitized":
        print(build_host_sanitized(verbose=True))
    else:
        print(build(verbose=True))
