"""CPU checks of the measurement script's accounting: the algorithmic flops and bytes the
bench lines divide by, the guard on measured HBM traffic taken on other kernel sources,
and the refusal of a multi-GPU run."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from gqa_attention_sink_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("lens_q,lens_kv,causal", [
    ([100, 37, 300], [100, 90, 300], True),     # with and without a cached prefix
    ([64, 1, 129], [64, 1, 129], True),
    ([50, 20], [70, 20], False),
    ([5], [3], True),                            # more queries than keys: early rows see none
])
def test_prefill_flops_match_oracle_count(lens_q, lens_kv, causal):
    w = wl.make_prefill(lens_q, lens_kv, 8, 2, 64, ("normal", 0, 1), 0.125, causal, seed=3,
                        device="cpu")
    assert bench.prefill_flops(w) == oracle.flops_causal(w.cu_seqlens_q, w.cu_seqlens_kv, w.hq,
                                                        w.d, causal)


def test_prefill_flops_closed_form():
    # one causal sequence of n queries over n keys: n(n+1)/2 visible pairs
    n = 6000
    assert bench._pairs([n], [n], True) == n * (n + 1) // 2
    assert bench._pairs([n], [n], False) == n * n


def test_decode_bytes_count_every_tensor():
    """K and V of every sequence once, Q read and the output written once (bf16), the
    fp32 lse, the sinks and kv_indptr; the first kernel alone writes no output or lse."""
    w = wl.make_decode([300, 1, 77, 4096], 4, 32, 4, 128, ("normal", 0, 2), 0.088, True, 0,
                       seed=5, device="cpu")
    kv = (w.k.numel() + w.v.numel()) * 2          # [Hkv, total_kv, D] bf16, no padding
    q = w.q.numel() * 2
    lse = w.batch * w.q_len * w.hq * 4
    small = w.sinks.numel() * 4 + w.cu_seqlens_kv.numel() * 4
    assert bench.decode_bytes(w) == kv + 2 * q + lse + small
    assert bench.decode_bytes(w, first_step_only=True) == kv + q + small


def test_traffic_only_for_current_sources(monkeypatch):
    """Measured traffic is reported only while the kernel sources hash to the value
    recorded with the counters."""
    import json
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    key = next(iter(rec))
    kernel, workload = key.split(":", 1)
    monkeypatch.setattr(bench, "_source_hash", lambda: rec[key]["source_hash"])
    assert bench._traffic_for(kernel, workload) == rec[key]["bytes_per_launch"]
    monkeypatch.setattr(bench, "_source_hash", lambda: "0" * 16)
    assert bench._traffic_for(kernel, workload) is None
    assert bench._traffic_for("no_such_kernel", workload) is None


def test_multi_gpu_run_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
