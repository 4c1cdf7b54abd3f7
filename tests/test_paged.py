"""GPU parity of the paged-KV path (decode over a paged HND cache, and the KV append
kernel) against the CPU oracle, through the C ABI.  Tolerances as in test_parity:
bf16 outputs max-abs <= 2e-2 and mean-abs <= 2e-3, lse within 1e-3; the append is a
copy and is checked bit for bit."""
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
    print(f"[paged] {msg}", flush=True)
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


def _run(sa, w, pk, ns=None):
    return sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,
                           pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale, w.causal,
                           w.num_splits if ns is None else ns)


def _oracle(w, pk):
    return oracle.sink_attention_decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks,
                                              pk.kv_page_indptr.cpu(), pk.kv_page_indices.cpu(),
                                              pk.kv_last_page_len.cpu(), pk.page_size, w.scale,
                                              w.causal)


def test_paged_decode_gptoss_full(sa):
    """The gpt-oss-like decode batch in a paged cache (page_size 16, pages scattered),
    every output checked against the oracle over the pages and against the contiguous
    definition."""
    w = wl.make("decode_gptoss", device="cuda")
    pk = wl.make_paged(w, 16, seed=77)
    _say(f"decode_gptoss paged ps=16 pages={pk.num_pages}")
    out, lse = _run(sa, w, pk)
    torch.cuda.synchronize()
    ro, rl = _oracle(w, pk)
    _compare(out, lse, ro, rl, "paged decode_gptoss")
    co, cl = oracle.sink_attention_decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, w.causal)
    assert np.array_equal(co, ro) and np.array_equal(cl, rl)


PAGED_CASES = [
    # lens_kv, q_len, hq, hkv, d, sink, causal, num_splits, page_size
    ([1, 2, 31, 33, 64], 1, 8, 1, 64, ("normal", 0, 2), True, 0, 16),
    ([5, 40, 1000], 4, 16, 4, 128, ("normal", 0, 2), True, 0, 16),
    ([4, 100, 777], 3, 8, 2, 64, ("alt_neginf", 2, 1), True, 3, 48),
    ([129, 2049], 2, 64, 8, 64, ("normal", 0, 2), True, 64, 32),
    ([600, 300], 4, 64, 2, 128, ("normal", 0, 2), True, 5, 64),       # 2 row groups
    ([512, 70], 1, 8, 8, 128, None, True, 1, 256),                     # one slot: direct
    ([90, 45], 4, 12, 4, 64, ("normal", 8, 1), False, 0, 16),
    ([3000, 4096, 16], 1, 64, 8, 64, ("normal", 0, 2), True, 0, 128),
    ([64, 48, 2], 2, 32, 2, 64, ("normal", 0, 2), True, 0, 16),        # 32 rows per KV head
]


@pytest.mark.parametrize("case", range(len(PAGED_CASES)))
def test_paged_decode_cases(sa, case):
    lens, ql, hq, hkv, d, sink, causal, ns, ps = PAGED_CASES[case]
    _say(f"case {case}: lens={lens} q_len={ql} hq={hq} hkv={hkv} d={d} ns={ns} ps={ps}")
    w = wl.make_decode(lens, ql, hq, hkv, d, sink, 1 / math.sqrt(d), causal, ns,
                       seed=500 + case, device="cuda")
    pk = wl.make_paged(w, ps, seed=600 + case)
    out, lse = _run(sa, w, pk)
    torch.cuda.synchronize()
    ro, rl = _oracle(w, pk)
    _compare(out, lse, ro, rl, f"paged case {case}")


def test_paged_unused_slots_do_not_leak(sa):
    """Cache slots no token occupies hold NaN: the output stays finite and equals the
    output over a cache whose spare slots hold random values, bit for bit."""
    w = wl.make_decode([17, 300, 1025, 33], 2, 16, 2, 64, ("normal", 0, 2), 0.125, True, 0,
                       seed=610, device="cuda")
    a = wl.make_paged(w, 32, seed=611, fill="nan")
    b = wl.make_paged(w, 32, seed=611, fill="randn")
    _say("NaN in unused slots")
    oa, la = _run(sa, w, a)
    ob, lb = _run(sa, w, b)
    torch.cuda.synchronize()
    assert torch.isfinite(oa.float()).all()
    assert torch.equal(oa, ob) and torch.equal(la, lb)


def test_paged_equals_contiguous_kernel_bitwise(sa):
    """With the same chunk plan (4 chunks forced on both sides) the paged and contiguous
    chunk kernels combine the same keys in the same order: identical results."""
    w = wl.make_decode([700, 3000, 64, 1], 1, 64, 8, 64, ("normal", 0, 2), 0.125, True, 0,
                       seed=620, device="cuda")
    pk = wl.make_paged(w, 64, seed=621)
    _say("paged vs contiguous chunk kernels")
    op, lp = _run(sa, w, pk, ns=4)
    po, pl = sa.decode_partial(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,
                               w.causal, 4)
    oc, lc = sa.merge(po, pl)
    torch.cuda.synchronize()
    assert torch.equal(op.reshape(oc.shape), oc) and torch.equal(lp.reshape(lc.shape), lc)


@pytest.mark.parametrize("ps,d,ql,hq,hkv", [(16, 64, 1, 64, 8), (32, 128, 2, 16, 4)])
def test_paged_stream_equals_contiguous_stream_bitwise(sa, ps, d, ql, hq, hkv):
    """Sequence lengths that are multiples of the page size make the page list, laid end
    to end, the same token axis as the contiguous cache: the stream plan, its ranges and
    the order of every sum are then the same, so paged and contiguous decode agree bit
    for bit although the pages are scattered."""
    lens = [704, 3008, ps, 4 * ps, 1536]
    w = wl.make_decode(lens, ql, hq, hkv, d, ("normal", 0, 2), 1 / math.sqrt(d), True, 0,
                       seed=630 + ps, device="cuda")
    pk = wl.make_paged(w, ps, seed=631 + ps, fill="nan")
    _say(f"paged vs contiguous stream decode ps={ps} d={d}")
    op, lp = _run(sa, w, pk)
    oc, lc = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, w.causal, 0)
    torch.cuda.synchronize()
    assert torch.isfinite(op.float()).all()
    assert torch.equal(op.reshape(oc.shape), oc) and torch.equal(lp.reshape(lc.shape), lc)


@pytest.mark.parametrize("ps,d,ql,hq,hkv", [(16, 128, 4, 32, 2), (48, 64, 3, 48, 4)])
def test_paged_whole_runs_equal_contiguous_bitwise(sa, ps, d, ql, hq, hkv):
    """Planner mode with more than 16 rows per KV head and a batch of nearly equal
    lengths that gives two workgroups per compute unit: paged and contiguous decode both
    take whole-sequence runs, the same chunks of every sequence in the same order, so
    they agree bit for bit (and with the oracle), although the pages are scattered and
    unused slots hold NaN."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    batch = -(-2 * cus // hkv)
    g = torch.Generator().manual_seed(650 + ps)
    lens = (480 + torch.randint(0, 33, (batch,), generator=g)).tolist()
    lens[3] = 0
    w = wl.make_decode(lens, ql, hq, hkv, d, ("normal", 0, 2), 1 / math.sqrt(d), True, 0,
                       seed=660 + ps, device="cuda")
    pk = wl.make_paged(w, ps, seed=661 + ps, fill="nan")
    entries = pk.kv_page_indices.numel()
    assert sa.decode_plan_kind(batch, ql, hq, hkv, d, (entries - batch) * ps, w.max_kv, 0) \
        == "whole_runs"
    assert sa.decode_plan_kind(batch, ql, hq, hkv, d, w.k.shape[1], w.max_kv, 0) == "whole_runs"
    _say(f"paged vs contiguous whole runs ps={ps} d={d} batch={batch}")
    op, lp = _run(sa, w, pk)
    oc, lc = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, w.causal, 0)
    torch.cuda.synchronize()
    assert torch.isfinite(op.float()).all()
    assert torch.equal(op.reshape(oc.shape), oc) and torch.equal(lp.reshape(lc.shape), lc)
    ro, rl = oracle.sink_attention_decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, w.causal)
    err = np.abs(op.float().cpu().numpy().astype(np.float64).reshape(ro.shape) - ro)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


@pytest.mark.parametrize("ps,d", [(16, 64), (48, 128), (256, 64)])
def test_kv_append_bitwise(sa, ps, d):
    """Append 1..37 new tokens per sequence into a scattered paged cache; the whole caches
    (including every slot that must not change) equal the oracle's append bit for bit."""
    g = torch.Generator().manual_seed(700 + ps)
    new = torch.randint(1, 38, (6,), generator=g).tolist()
    new[2] = 0                                          # a sequence with nothing to append
    old = torch.randint(0, 300, (6,), generator=g).tolist()
    full = [o + n for o, n in zip(old, new)]
    hkv = 4
    w = wl.make_decode(full, 1, hkv, hkv, d, None, 0.1, True, 0, seed=710 + ps, device="cuda")
    pk = wl.make_paged(w, ps, seed=720 + ps)
    kc0, vc0 = pk.k_cache.clone(), pk.v_cache.clone()
    gk = wl._gen("cuda", 730 + ps)
    k_new = wl._randn_bf16((sum(new), hkv, d), gk, "cuda")
    v_new = wl._randn_bf16((sum(new), hkv, d), gk, "cuda")
    app = torch.tensor([0] + np.cumsum(new).tolist(), dtype=torch.int32, device="cuda")
    _say(f"append ps={ps} d={d} new={new}")
    sa.kv_append(k_new, v_new, app, pk.kv_page_indptr, pk.kv_page_indices, pk.kv_last_page_len,
                 pk.k_cache, pk.v_cache, max(new))
    torch.cuda.synchronize()
    rk, rv = oracle.kv_append(kc0, vc0, k_new, v_new, app.cpu(), pk.kv_page_indptr.cpu(),
                              pk.kv_page_indices.cpu(), pk.kv_last_page_len.cpu(), ps)
    assert np.array_equal(_np(pk.k_cache), rk)
    assert np.array_equal(_np(pk.v_cache), rv)


def test_append_then_decode(sa):
    """One decode step of an engine: append this step's q_len keys/values to the paged
    cache, then attend; equals the oracle over the full contiguous KV."""
    ql, hq, hkv, d, ps = 2, 32, 4, 64, 16
    w = wl.make_decode([50, 513, 2048, 7], ql, hq, hkv, d, ("normal", 0, 2), 0.125, True, 0,
                       seed=740, device="cuda")
    pk = wl.make_paged(w, ps, seed=741)
    # the newest q_len tokens of every sequence are overwritten with garbage, then appended
    ind = w.cu_seqlens_kv.tolist()
    rows = torch.cat([torch.arange(ind[b + 1] - ql, ind[b + 1]) for b in range(w.batch)]).cuda()
    k_new = w.k[:, rows].permute(1, 0, 2).contiguous()
    v_new = w.v[:, rows].permute(1, 0, 2).contiguous()
    page_of = pk.kv_page_indices.tolist()
    indptr = pk.kv_page_indptr.tolist()
    for b in range(w.batch):
        lk = w.lens_kv[b]
        for t in range(lk - ql, lk):
            page = page_of[indptr[b] + t // ps]
            pk.k_cache[page, :, t % ps] = float("nan")
            pk.v_cache[page, :, t % ps] = float("nan")
    app = torch.arange(w.batch + 1, dtype=torch.int32, device="cuda") * ql
    _say("append then decode")
    sa.kv_append(k_new, v_new, app, pk.kv_page_indptr, pk.kv_page_indices, pk.kv_last_page_len,
                 pk.k_cache, pk.v_cache, ql)
    out, lse = _run(sa, w, pk)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, w.causal)
    _compare(out, lse, ro, rl, "append+decode")
