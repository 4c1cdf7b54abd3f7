"""The host side of the C ABI (argument validation, the decode and prefill planners,
workspace sizing) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and exercised by the CPU ABI and plan tests.

The sanitized library is api.cpp linked against a stub launch layer that reports no
device, so every host path runs as in the HIP library and a valid call ends in
SINK_ATTN_ERR_HIP where the library would launch.  The test suites run in a child
process with the sanitizer runtimes preloaded (the Python interpreter is not
instrumented) and the binding pointed at the sanitized build; any sanitizer report
aborts that process and fails this test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs g++ with the sanitizer runtimes")
def test_host_code_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not installed")
    sys.path.insert(0, ROOT)
    from gqa_attention_sink_amd.build import build_host_sanitized
    lib = build_host_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", SINK_ATTN_LIB=lib)
    probe = ("from gqa_attention_sink_amd import sink_attn as s; "
             "assert s.LIB_PATH == %r, s.LIB_PATH; s.load(); print('loaded', s.LIB_PATH)" % lib)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", "tests/test_abi.py", "tests/test_decode_stream.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error" not in out
