"""GPU parity of the key-split prefill (chunked prefill over a cached prefix and other
under-filled grids): splits of the key axis, the sink in split 0 only, merged by
log-sum-exp, against the fp64 oracle.  Tolerances as in test_parity."""
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
    print(f"[prefill-split] {msg}", flush=True)
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


def _compare(out, lse, ro, rl, what):
    o = _np(out).reshape(ro.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ro)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    l = _np(lse).reshape(rl.shape)
    assert np.array_equal(np.isneginf(l), np.isneginf(rl)), f"{what}: -inf lse pattern"
    fin = np.isfinite(rl)
    if fin.any():
        assert np.abs(l[fin] - rl[fin]).max() <= LSE_TOL, f"{what}: lse"


def _run(sa, w, ns):
    return sa.prefill(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q, w.cu_seqlens_kv, w.max_q, w.scale,
                      w.causal, num_splits=ns, max_seqlen_kv=w.max_kv)


CASES = [
    # lens_q, lens_kv, hq, hkv, d, sink, causal, num_splits
    ([200, 37, 513], [900, 37, 2000], 16, 4, 64, ("normal", 0, 2), True, 0),
    ([200, 37, 513], [900, 37, 2000], 16, 4, 64, ("normal", 0, 2), True, 5),
    ([64, 1, 300], [4000, 1, 300], 8, 2, 128, ("alt_neginf", 2, 1), True, 3),
    ([100, 50], [3000, 700], 12, 4, 64, ("normal", 8, 1), False, 4),
    ([128, 0, 17], [6000, 9, 17], 8, 8, 128, ("normal", 0, 2), True, 16),   # empty query seq
    ([1, 1], [5000, 1], 64, 8, 64, None, True, 0),                            # decode-like rows
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_prefill_split_cases(sa, case):
    lq, lk, hq, hkv, d, sink, causal, ns = CASES[case]
    w = wl.make_prefill(lq, lk, hq, hkv, d, sink, 1 / math.sqrt(d), causal, seed=900 + case,
                        device="cuda")
    s = sa.prefill_num_splits(w.batch, w.max_q, w.max_kv, hq, hkv, ns)
    _say(f"case {case}: lq={lq} lk={lk} hq={hq} hkv={hkv} d={d} ns={ns} -> {s} splits")
    assert s >= 2
    out, lse = _run(sa, w, ns)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q.cpu(),
                                   w.cu_seqlens_kv.cpu(), w.scale, w.causal)
    _compare(out, lse, ro, rl, f"split case {case}")


def test_split_invariance(sa):
    w = wl.make_prefill([300, 77], [2500, 77], 16, 2, 64, ("normal", 0, 2), 0.125, True,
                        seed=950, device="cuda")
    _say("split invariance")
    ro, rl = oracle.sink_attention(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q.cpu(),
                                   w.cu_seqlens_kv.cpu(), w.scale, w.causal)
    for ns in (1, 2, 7, 40):
        out, lse = _run(sa, w, ns)
        torch.cuda.synchronize()
        _compare(out, lse, ro, rl, f"num_splits={ns}")


@pytest.mark.slow
def test_chunked_prefill_full_sampled(sa):
    """The chunked-prefill workload at full size with the planner's splits; sampled rows
    (each against the oracle over exactly the keys it sees)."""
    w = wl.make("chunked_prefill", device="cuda")
    s = sa.prefill_num_splits(w.batch, w.max_q, w.max_kv, w.hq, w.hkv, 0)
    _say(f"chunked_prefill full: lq={w.lens_q} lk={w.lens_kv} splits={s}")
    assert s > 1
    out, lse = _run(sa, w, 0)
    torch.cuda.synchronize()
    cq = w.cu_seqlens_q.cpu().tolist()
    ck = w.cu_seqlens_kv.cpu().tolist()
    for b in range(w.batch):
        lq, lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        for i in (0, 1, 63, 64, 511, lq - 1):
            nk = i + (lk - lq) + 1
            ro, rl = oracle.sink_attention(w.q[cq[b] + i:cq[b] + i + 1], w.k[:, ck[b]:ck[b] + nk],
                                           w.v[:, ck[b]:ck[b] + nk], w.sinks, [0, 1], [0, nk],
                                           w.scale, True)
            _compare(out[cq[b] + i:cq[b] + i + 1], lse[cq[b] + i:cq[b] + i + 1], ro, rl,
                     f"chunked b={b} i={i}")
