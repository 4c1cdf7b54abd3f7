"""Element-wise parity at the full sizes the bench measures: every output and lse of the
varlen prefill (8 sequences of 512..6000 tokens, 64 query heads over 8, head_dim 64),
the 6000-token prefill over 4 KV heads (head_dim 128, half the heads with a -inf sink),
the chunked prefill (1024 new tokens over a 31744-token prefix, key splits from the
planner), and all 256 sequences of the speculative decode (4 draft tokens over 32768
keys) through its three paths: 32 chunks per sequence as the workload names them, the
planner (whole-sequence runs: equal lengths and at least two workgroups per compute
unit), and the stream plan's two steps on their own (equal ranges of each head's token
axis, merged with the sinks).  These are the workloads of "Hosting Qwen on Blackwell"
(Prefillers: ~6000-token inputs over 4 KV heads; Decoders: large batches, MTP draft
tokens).

The oracle runs unchanged: prefill in parallel CPU processes over independent
(sequence, KV head, row block) pieces (tests/_oracle_pool.py), decode one sequence at a
time with that sequence's K/V copied to the host.  Tolerances as everywhere: out
max-abs <= 2e-2 and mean-abs <= 2e-3, lse <= 1e-3, -inf lse exactly.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import _oracle_pool
from gqa_attention_sink_amd import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

MAX_ABS, MEAN_ABS, LSE_TOL = 2e-2, 2e-3, 1e-3


def _say(msg):
    print(f"[full] {msg}", flush=True)
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


def _f32(t):
    return t.detach().float().cpu().numpy()


def _compare(out, lse, ref_out, ref_lse, what):
    o = _np(out).reshape(ref_out.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ref_out)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    l = _np(lse).reshape(ref_lse.shape)
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse)), f"{what}: -inf lse pattern"
    fin = np.isfinite(ref_lse)
    le = np.abs(l[fin] - ref_lse[fin]).max() if fin.any() else 0.0
    assert le <= LSE_TOL, f"{what}: lse err {le:.3e}"
    return err.max(), err.mean(), le


def _prefill_full(sa, name, num_splits=1):
    w = wl.make(name, device="cuda")
    if num_splits == 0:  # the planner must split this workload's key axis
        assert sa.prefill_num_splits(w.batch, w.max_q, w.max_kv, w.hq, w.hkv, 0) > 1
    _say(f"{name}: lens_q={w.lens_q} lens_kv={w.lens_kv} splits={num_splits}")
    out, lse = sa.prefill(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q, w.cu_seqlens_kv, w.max_q,
                          w.scale, w.causal, num_splits=num_splits, max_seqlen_kv=w.max_kv)
    torch.cuda.synchronize()
    ro, rl = _oracle_pool.prefill_reference(
        _f32(w.q), _f32(w.k), _f32(w.v), None if w.sinks is None else _f32(w.sinks),
        w.cu_seqlens_q.cpu().tolist(), w.cu_seqlens_kv.cpu().tolist(), w.scale, w.causal)
    r = _compare(out, lse, ro, rl, name)
    _say(f"{name}: max-abs {r[0]:.2e} mean-abs {r[1]:.2e} lse {r[2]:.2e}")


def test_varlen_prefill_full_elementwise(sa):
    _prefill_full(sa, "varlen_prefill")


def test_long_prefill_full_elementwise(sa):
    _prefill_full(sa, "long_prefill")


def test_chunked_prefill_full_elementwise(sa):
    _prefill_full(sa, "chunked_prefill", num_splits=0)


def test_spec_decode_full_every_sequence(sa):
    """All 256 sequences, every draft token and head, through the 32-chunk path (runs of
    chunks merged in the workgroup), the planner (whole-sequence runs) and the stream
    plan's partial and merge steps (decode_stream_wg_kernel with 4 wavefronts)."""
    w = wl.make("spec_decode", device="cuda")
    tk = w.k.shape[1]
    assert w.num_splits == 32
    assert sa.decode_plan_kind(w.batch, w.q_len, w.hq, w.hkv, w.d, tk, w.max_kv, 0) == "whole_runs"
    assert sa.decode_plan_kind(w.batch, w.q_len, w.hq, w.hkv, w.d, tk, w.max_kv, 32) == "chunks"
    assert sa.decode_stream_plan(w.batch, w.q_len, w.hq, w.hkv, w.d, tk, w.max_kv) is not None
    cps = sa.decode_chunks_per_slot(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, 32)
    _say(f"spec_decode full: 32 chunks ({cps} per workgroup), whole runs, stream steps")
    o32, l32 = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, w.causal, 32)
    owr, lwr = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, w.causal, 0)
    _, _, ws = sa.decode_stream_partial(w.q, w.k, w.v, w.cu_seqlens_kv, w.max_kv, w.scale, w.causal)
    ost, lst = sa.decode_stream_merge(w.sinks, w.cu_seqlens_kv, tuple(w.q.shape), tk, w.hkv,
                                      w.max_kv, ws)
    torch.cuda.synchronize()
    ind = w.cu_seqlens_kv.cpu().tolist()
    worst = np.zeros(3)
    for b in range(w.batch):
        ks = slice(ind[b], ind[b + 1])
        ro, rl = oracle.sink_attention_decode(w.q[b:b + 1], w.k[:, ks], w.v[:, ks], w.sinks,
                                              [0, ind[b + 1] - ind[b]], w.scale, w.causal)
        for out, lse, what in ((o32, l32, "32 chunks"), (owr, lwr, "whole runs"),
                               (ost, lst, "stream steps")):
            r = _compare(out[b:b + 1], lse[b:b + 1], ro, rl, f"spec_decode {what} b={b}")
            worst = np.maximum(worst, r)
    _say(f"spec_decode full: worst max-abs {worst[0]:.2e} mean-abs {worst[1]:.2e} lse {worst[2]:.2e}")
