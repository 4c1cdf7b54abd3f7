"""HIP graph capture of the entry points: every call enqueues kernels on the caller's stream
and nothing else (no allocation, no memset, no synchronisation), so a captured call
replays to the eager result.  Each graph is replayed several times with eager work
between the replays (the outputs are cleared by a fill kernel and the caches
re-written), and every replay is compared bit for bit with the eager call.
"""
import math
import sys

import pytest
import torch

from gqa_attention_sink_amd import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _say(msg):
    print(f"[graph] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sink_amd as pkg
    pkg.load()
    return pkg


def _capture(fn):
    """Warm up on a side stream (first-call lookups happen there), then capture fn."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, outs, refs, what, between=None):
    for i in range(REPLAYS):
        for o in outs:
            o.zero_()               # eager work between replays (a fill kernel)
        if between is not None:
            between()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"{what}: replay {i} differs from the eager call"


@pytest.mark.parametrize("ns", [0, 5])
def test_graph_decode(sa, ns):
    """Planner (stream plan: partial kernel + merge) and forced chunks (split + merge)."""
    w = wl.make_decode([700, 3000, 64, 1, 2100], 2, 16, 4, 64, ("normal", 0, 2), 0.125, True,
                       ns, seed=1100 + ns, device="cuda")
    _say(f"decode ns={ns}: plan {sa.decode_plan_kind(5, 2, 16, 4, 64, w.k.shape[1], w.max_kv, ns)}")
    ws = sa.decode_workspace(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, ns)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.q_len, w.hq), dtype=torch.float32, device="cuda")
    call = lambda: sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,  # noqa: E731
                             w.causal, ns, workspace=ws, out=out, lse=lse)
    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = _capture(call)
    _replay_and_check(g, [out, lse], [ref_o, ref_l], f"decode ns={ns}")


def test_graph_decode_noalloc(sa):
    w = wl.make_decode([900, 40, 2500], 1, 64, 8, 64, ("normal", 0, 2), 0.125, True, 0,
                       seed=1110, device="cuda")
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.q_len, w.hq), dtype=torch.float32, device="cuda")
    call = lambda: sa.decode_noalloc(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, out,  # noqa: E731
                                     lse, sm_scale=w.scale, causal=w.causal)
    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = _capture(call)
    _replay_and_check(g, [out, lse], [ref_o, ref_l], "decode_noalloc")


@pytest.mark.parametrize("d,ns", [(128, 1), (64, 1), (64, 3)])
def test_graph_prefill(sa, d, ns):
    """The ping-pong (D=128) and lock-step (D=64) kernels, and a key-split prefill with
    its merge."""
    w = wl.make_prefill([300, 77], [300 + 128 * (ns > 1), 77], 16, 4, d, ("alt_neginf", 2, 1),
                        1 / math.sqrt(d), True, seed=1120 + d + ns, device="cuda")
    out = torch.empty_like(w.q)
    lse = torch.empty((w.q.shape[0], w.hq), dtype=torch.float32, device="cuda")
    ws = None
    if ns > 1:
        ws = torch.empty(max(256, sa.prefill_workspace_bytes(w.q.shape[0], w.hq, d, ns)),
                         dtype=torch.uint8, device="cuda")
    call = lambda: sa.prefill(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q, w.cu_seqlens_kv,  # noqa: E731
                              w.max_q, w.scale, w.causal, out=out, lse=lse, num_splits=ns,
                              max_seqlen_kv=w.max_kv, workspace=ws)
    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = _capture(call)
    _replay_and_check(g, [out, lse], [ref_o, ref_l], f"prefill d={d} ns={ns}")


def test_graph_paged_append_then_decode(sa):
    """A captured step that appends new K/V into a paged cache and decodes over it; the
    eager work between replays restores the cache, so every replay repeats the append."""
    w = wl.make_decode([512, 96, 1000], 1, 32, 4, 128, ("normal", 0, 2), 1 / math.sqrt(128), True,
                       0, seed=1130, device="cuda")
    pk = wl.make_paged(w, 32, seed=1131)
    kc_full, vc_full = pk.k_cache.clone(), pk.v_cache.clone()
    # the last 5 tokens of each sequence are the "new" ones the step appends
    new = 5
    starts = w.cu_seqlens_kv.tolist()
    rows = [t for b in range(w.batch) for t in range(starts[b + 1] - new, starts[b + 1])]
    idx = torch.tensor(rows, device="cuda")
    k_new = w.k[:, idx].permute(1, 0, 2).contiguous()
    v_new = w.v[:, idx].permute(1, 0, 2).contiguous()
    app = torch.arange(0, (w.batch + 1) * new, new, dtype=torch.int32, device="cuda")
    ws = sa.decode_workspace(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, 0)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.q_len, w.hq), dtype=torch.float32, device="cuda")

    def step():
        sa.kv_append(k_new, v_new, app, pk.kv_page_indptr, pk.kv_page_indices,
                     pk.kv_last_page_len, pk.k_cache, pk.v_cache, new)
        sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,
                        pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale, w.causal, 0,
                        workspace=ws, out=out, lse=lse)

    # the cache before the step: the new tokens' slots hold zeros (an append of zeros)
    sa.kv_append(torch.zeros_like(k_new), torch.zeros_like(v_new), app, pk.kv_page_indptr,
                 pk.kv_page_indices, pk.kv_last_page_len, pk.k_cache, pk.v_cache, new)
    kc0, vc0 = pk.k_cache.clone(), pk.v_cache.clone()
    assert not torch.equal(kc0, kc_full)

    def restore():
        pk.k_cache.copy_(kc0)
        pk.v_cache.copy_(vc0)

    step()
    torch.cuda.synchronize()
    assert torch.equal(pk.k_cache, kc_full) and torch.equal(pk.v_cache, vc_full)
    ref_o, ref_l = out.clone(), lse.clone()
    restore()
    g = _capture(step)
    _replay_and_check(g, [out, lse], [ref_o, ref_l], "paged append + decode", between=restore)
    assert torch.equal(pk.k_cache, kc_full) and torch.equal(pk.v_cache, vc_full)
