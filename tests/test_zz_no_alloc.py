"""The no-allocation decode entry point (sink_attn_decode_noalloc) against
sink_attn_decode: same plan and kernels, the partials in the library's per-GPU scratch
array instead of a caller's workspace.  Two calls in a row, the second with a smaller
input, each compared with sink_attn_decode bit for bit and with the fp64 oracle to the
parity tolerance; then the forced-chunk path (more than 16 rows per KV head) likewise."""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from gqa_attention_sink_amd import workloads as wl

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_TOL = 2e-2, 2e-3, 1e-3


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sink_amd as pkg
    pkg.load()
    return pkg


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_against_decode(sa, w, num_splits):
    ws = sa.decode_workspace_bytes(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, num_splits)
    assert 0 < ws <= sa.decode_noalloc_scratch_bytes()
    ref_out, ref_lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,
                                 w.causal, num_splits)
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((w.batch, w.q_len, w.hq), float("nan"), dtype=torch.float32,
                     device=w.q.device)
    sa.decode_noalloc(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, out, lse, w.scale,
                      w.causal, num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "out differs"
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32)), "lse differs"
    ro, rl = oracle.sink_attention_decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, w.causal)
    o = _np(out).reshape(ro.shape)
    err = np.abs(o - ro)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
    l = _np(lse).reshape(rl.shape)
    assert np.array_equal(np.isneginf(l), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.abs(l[fin] - rl[fin]).max() <= LSE_TOL


@pytest.mark.parametrize("case", [
    # (first call, second smaller call): lens, q_len, hq, hkv, d, num_splits
    (([1024, 8192, 3000, 5000, 7777, 2048, 4096, 1500] * 2, 1, 64, 8, 64, 0),
     ([900, 4000, 31, 0, 2500], 1, 64, 8, 64, 0)),
    (([4096, 1000, 33, 2900, 4100, 700], 4, 64, 4, 128, 8),
     ([640, 50, 1], 4, 64, 4, 128, 8)),
])
def test_noalloc_matches_decode_twice(sa, case):
    for i, (lens, ql, hq, hkv, d, ns) in enumerate(case):
        _say(f"call {i}: lens={lens} q_len={ql} hq={hq} hkv={hkv} d={d} ns={ns}")
        w = wl.make_decode(lens, ql, hq, hkv, d, ("normal", 0, 2), 1 / math.sqrt(d), True, ns,
                           seed=900 + 10 * i + ql, device="cuda")
        _check_against_decode(sa, w, ns)


def test_noalloc_whole_runs_need_no_scratch(sa):
    """A batch that takes whole-sequence runs needs more than the array as a workspace for
    the other plans, yet runs: those runs write no partials.  Bit for bit against
    sink_attn_decode, then a smaller call through the array."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    batch = -(-2 * cus // 2)
    g = torch.Generator().manual_seed(960)
    lens = (480 + torch.randint(0, 33, (batch,), generator=g)).tolist()
    w = wl.make_decode(lens, 4, 32, 2, 128, ("normal", 0, 2), 1 / math.sqrt(128), True, 0,
                       seed=961, device="cuda")
    assert sa.decode_plan_kind(batch, 4, 32, 2, 128, w.k.shape[1], w.max_kv, 0) == "whole_runs"
    assert sa.decode_workspace_bytes(batch, 4, 32, 2, 128, w.max_kv, 0) > \
        sa.decode_noalloc_scratch_bytes()
    _say(f"whole runs through the no-allocation entry point: batch={batch}")
    ref_out, ref_lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,
                                 True, 0)
    out = torch.full_like(w.q, float("nan"))
    lse = torch.full((batch, 4, 32), float("nan"), dtype=torch.float32, device="cuda")
    sa.decode_noalloc(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, out, lse, w.scale,
                      True, 0)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
    small = wl.make_decode([300, 2000, 7], 1, 64, 8, 64, ("normal", 0, 2), 0.125, True, 0,
                           seed=962, device="cuda")
    _check_against_decode(sa, small, 0)


def test_noalloc_rejects_oversize(sa):
    """64 sequences of 4 draft tokens over 64 query heads (16384 rows) need a 142 MB
    workspace, more than the array holds: a clear error before any launch, and the
    entry point keeps working afterwards."""
    big = wl.make_decode([64] * 64, 4, 64, 4, 128, ("normal", 0, 2), 1 / math.sqrt(128), True,
                         0, seed=950, device="cuda")
    assert sa.decode_workspace_bytes(64, 4, 64, 4, 128, 64, 0) > sa.decode_noalloc_scratch_bytes()
    out = torch.empty_like(big.q)
    with pytest.raises(sa.SinkAttnError, match="SCRATCH_LIMIT"):
        sa.decode_noalloc(big.q, big.k, big.v, big.sinks, big.cu_seqlens_kv, big.max_kv, out,
                          None, big.scale, True, 0)
    w = wl.make_decode([64, 700, 3], 4, 64, 4, 128, ("normal", 0, 2), 1 / math.sqrt(128), True,
                       0, seed=951, device="cuda")
    _check_against_decode(sa, w, 0)
