"""Calls from several host threads, each on its own stream with its own workspace and
outputs: the library keeps no per-call state (only the per-device compute-unit count,
read once), so concurrent calls give the results of the same calls made one by one.
"""
import math
import sys
import threading

import pytest
import torch

from gqa_attention_sink_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sink_amd as pkg
    pkg.load()
    return pkg


def test_threads_and_streams(sa):
    print("[concurrency] 4 threads x 3 calls, decode and prefill", flush=True)
    sys.stdout.flush()
    works = []
    for i in range(4):
        if i % 2 == 0:
            w = wl.make_decode([600 + 100 * i, 2500, 31, 1800], 2, 32, 4, 128, ("normal", 0, 2),
                               1 / math.sqrt(128), True, 0, seed=1200 + i, device="cuda")
            ws = sa.decode_workspace(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, 0)
            out = torch.empty_like(w.q)
            call = (lambda w=w, ws=ws, out=out:
                    sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,
                              w.causal, 0, workspace=ws, out=out)[0])
        else:
            w = wl.make_prefill([400, 90], [700, 90], 16, 4, 64, ("alt_neginf", 2, 1), 0.125,
                                True, seed=1200 + i, device="cuda")
            out = torch.empty_like(w.q)
            call = (lambda w=w, out=out:
                    sa.prefill(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q, w.cu_seqlens_kv, w.max_q,
                               w.scale, w.causal, out=out)[0])
        works.append((call, out))
    refs = []
    for call, out in works:           # one by one, on the default stream
        call()
        torch.cuda.synchronize()
        refs.append(out.clone())
    errors = []

    def worker(j):
        try:
            call, out = works[j]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    out.zero_()
                    call()
                s.synchronize()
            if not torch.equal(out, refs[j]):
                errors.append(f"thread {j}: result differs")
        except Exception as e:  # noqa: BLE001
            errors.append(f"thread {j}: {e!r}")

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(len(works))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
