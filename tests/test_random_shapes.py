"""GPU parity on seeded random shapes: decode over contiguous and paged caches (every plan
the library picks for them: chunk runs, stream ranges, forced chunk counts) and prefill
with and without key splits, against the fp64 oracle.

Each case draws its batch, draft length, GQA group, KV heads, head_dim, per-sequence
lengths (some empty, some a single key, ragged against the 32-key stages and the
pages), sink kind, causal flag and chunk count from its own seed, so a failure names a
case that reruns alone.  Tolerances as everywhere: out max-abs <= 2e-2 and mean-abs
<= 2e-3, lse within 1e-3, -inf lse entries exactly.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from _rope_slack import decode_lse_slack, prefill_lse_slack
from gqa_attention_sink_amd import workloads as wl

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_TOL = 2e-2, 2e-3, 1e-3
SINKS = [("normal", 0, 2), ("alt_neginf", 2, 1), None, ("normal", 6, 1)]


def _say(msg):
    print(f"[random] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sink_amd as pkg
    pkg.load()
    return pkg


def _compare(out, lse, ref_out, ref_lse, what, lse_slack=None):
    o = out.detach().float().cpu().numpy().astype(np.float64).reshape(ref_out.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ref_out)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    l = lse.detach().float().cpu().numpy().astype(np.float64).reshape(ref_lse.shape)
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse)), f"{what}: -inf lse pattern"
    fin = np.isfinite(ref_lse)
    if fin.any():
        tol = LSE_TOL if lse_slack is None else LSE_TOL + np.asarray(lse_slack).reshape(ref_lse.shape)[fin]
        le = np.abs(l[fin] - ref_lse[fin])
        assert np.all(le <= tol), f"{what}: lse err {le.max():.3e} (worst over tolerance " \
                                  f"{np.max(le - tol):.3e})"


def _decode_case(i):
    r = np.random.default_rng(900 + i)
    ql = int(r.integers(1, 5))
    group = int(r.choice([1, 2, 4, 6, 8, 16]))
    hkv = int(r.choice([1, 2, 4, 8]))
    d = int(r.choice([64, 128]))
    batch = int(r.integers(1, 10))
    lens = [int(x) for x in r.integers(ql, 2600, batch)]
    ns = int(r.choice([0, 0, 0, 0, 1, 3, 7, 16]))
    sink = SINKS[int(r.integers(0, len(SINKS)))]
    causal = bool(r.integers(0, 4) > 0)
    if batch > 2:  # an empty sequence, or one with as many keys as draft tokens (or 1)
        lens[int(r.integers(0, batch))] = int(r.choice([0, ql] if causal else [0, 1, ql]))
    page = int(r.choice([0, 0, 0, 0, 16, 32, 64, 128]))   # 0: contiguous cache
    if 40 <= i < 44:  # the stream plan's workgroup kernel: planner, contiguous, 16 < rows <= 64
        ql, page, ns = 4, 0, 0
        group = [6, 8, 16, 16][i - 40]
    return lens, ql, group * hkv, hkv, d, sink, causal, ns, page


@pytest.mark.parametrize("i", range(44))
def test_random_decode(sa, i):
    lens, ql, hq, hkv, d, sink, causal, ns, page = _decode_case(i)
    w = wl.make_decode(lens, ql, hq, hkv, d, sink, 1 / math.sqrt(d), causal, ns,
                       seed=950 + i, device="cuda")
    kind = sa.decode_plan_kind(len(lens), ql, hq, hkv, d, w.k.shape[1], w.max_kv, ns)
    _say(f"decode {i}: lens={lens} q_len={ql} hq={hq} hkv={hkv} d={d} splits={ns} "
         f"sink={sink} causal={causal} page={page} plan={kind}")
    if page:
        pk = wl.make_paged(w, page, seed=960 + i, fill="nan")
        out, lse = sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,
                                   pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale,
                                   w.causal, ns)
    else:
        out, lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,
                             w.causal, ns)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, w.causal)
    _compare(out, lse, ro, rl, f"decode case {i}")


def _prefill_case(i):
    r = np.random.default_rng(1900 + i)
    group = int(r.choice([1, 2, 3, 4, 8, 16]))
    hkv = int(r.choice([1, 2, 4]))
    d = int(r.choice([64, 128]))
    batch = int(r.integers(1, 5))
    lens_q = [int(x) for x in r.integers(1, 700, batch)]
    prefix = [int(x) for x in r.integers(0, 600, batch)] if r.integers(0, 2) else [0] * batch
    lens_kv = [a + b for a, b in zip(lens_q, prefix)]
    ns = int(r.choice([1, 1, 0, 2, 5]))
    sink = SINKS[int(r.integers(0, len(SINKS)))]
    causal = bool(r.integers(0, 4) > 0)
    return lens_q, lens_kv, group * hkv, hkv, d, sink, causal, ns


@pytest.mark.parametrize("i", range(12))
def test_random_prefill(sa, i):
    lens_q, lens_kv, hq, hkv, d, sink, causal, ns = _prefill_case(i)
    _say(f"prefill {i}: lens_q={lens_q} lens_kv={lens_kv} hq={hq} hkv={hkv} d={d} "
         f"splits={ns} sink={sink} causal={causal}")
    w = wl.make_prefill(lens_q, lens_kv, hq, hkv, d, sink, 1 / math.sqrt(d), causal,
                        seed=1950 + i, device="cuda")
    out, lse = sa.prefill(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q, w.cu_seqlens_kv,
                          max(lens_q), w.scale, w.causal, num_splits=ns,
                          max_seqlen_kv=max(lens_kv))
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q.cpu(),
                                   w.cu_seqlens_kv.cpu(), w.scale, w.causal)
    _compare(out, lse, ro, rl, f"prefill case {i}")


# ---------------------------------------------------------------- with fused YaRN rotation
YARN = dict(theta=150000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0, beta_slow=1.0)
PLAIN = dict(theta=10000.0, factor=1.0, original_max_pos=4096, beta_fast=32.0, beta_slow=1.0)


def _rotated_q_decode(w, params):
    """The oracle's rotation of each query at its position Lk - q_len + t, rounded to bf16
    as the kernels' rotated operands are."""
    lens = np.array(w.lens_kv)
    pos = (lens[:, None] - w.q_len + np.arange(w.q_len)[None, :])[:, :, None]
    return oracle.bf16_round(oracle.apply_rope(w.q, pos, **params))


@pytest.mark.parametrize("i", range(16))
def test_random_decode_rope(sa, i):
    """Every decode plan with the query rotation fused into its Q loads."""
    lens, ql, hq, hkv, d, sink, causal, ns, page = _decode_case(100 + i)
    params = YARN if i % 4 else PLAIN
    w = wl.make_decode(lens, ql, hq, hkv, d, sink, 1 / math.sqrt(d), causal, ns,
                       seed=1050 + i, device="cuda")
    kind = sa.decode_plan_kind(len(lens), ql, hq, hkv, d, w.k.shape[1], w.max_kv, ns)
    _say(f"decode rope {i}: lens={lens} q_len={ql} hq={hq} hkv={hkv} d={d} splits={ns} "
         f"sink={sink} causal={causal} page={page} plan={kind} factor={params['factor']}")
    rope = sa.RopeParams(**params)
    if page:
        pk = wl.make_paged(w, page, seed=1060 + i, fill="nan")
        out, lse = sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,
                                   pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale,
                                   w.causal, ns, rope=rope)
    else:
        out, lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,
                             w.causal, ns, rope=rope)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_decode(_rotated_q_decode(w, params), w.k, w.v, w.sinks,
                                          w.cu_seqlens_kv.cpu(), w.scale, w.causal)
    slack = decode_lse_slack(w.q, w.lens_kv, params, w.k, w.cu_seqlens_kv, hq, hkv, w.scale,
                             w.causal)
    _compare(out, lse, ro, rl, f"decode rope case {i}", slack)


@pytest.mark.parametrize("page", [0, 32])
def test_whole_runs_rope(sa, page):
    """Whole-sequence runs (a batch that fills the GPU with nearly equal lengths) with the
    query rotation, on a contiguous and a paged cache."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    batch = -(-2 * cus // 2)  # 4 draft tokens x 8 heads per KV head, 2 KV heads: one row group
    g = torch.Generator().manual_seed(1070 + page)
    # lengths within 3 % of each other, long enough that the paged bound (page-list entries
    # less one page per sequence) still shows them nearly equal
    lens = (2000 + torch.randint(0, 65, (batch,), generator=g)).tolist()
    w = wl.make_decode(lens, 4, 16, 2, 128, ("normal", 0, 2), 1 / math.sqrt(128), True, 0,
                       seed=1071 + page, device="cuda")
    total = w.k.shape[1]
    rope = sa.RopeParams(**YARN)
    if page:
        pk = wl.make_paged(w, page, seed=1072, fill="nan")
        total = (pk.kv_page_indices.numel() - batch) * page
        out, lse = sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,
                                   pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale,
                                   True, 0, rope=rope)
    else:
        out, lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, True,
                             0, rope=rope)
    assert sa.decode_plan_kind(batch, 4, 16, 2, 128, total, w.max_kv, 0) == "whole_runs"
    _say(f"whole runs with rope: batch={batch} page={page}")
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_decode(_rotated_q_decode(w, YARN), w.k, w.v, w.sinks,
                                          w.cu_seqlens_kv.cpu(), w.scale, True)
    slack = decode_lse_slack(w.q, w.lens_kv, YARN, w.k, w.cu_seqlens_kv, 16, 2, w.scale, True)
    _compare(out, lse, ro, rl, f"whole runs rope page={page}", slack)


@pytest.mark.parametrize("i", range(6))
def test_random_prefill_rope(sa, i):
    """Prefill with and without key splits, with the query rotation at Lk - Lq + i."""
    lens_q, lens_kv, hq, hkv, d, sink, causal, ns = _prefill_case(100 + i)
    params = YARN if i % 3 else PLAIN
    _say(f"prefill rope {i}: lens_q={lens_q} lens_kv={lens_kv} hq={hq} hkv={hkv} d={d} "
         f"splits={ns} sink={sink} causal={causal} factor={params['factor']}")
    w = wl.make_prefill(lens_q, lens_kv, hq, hkv, d, sink, 1 / math.sqrt(d), causal,
                        seed=1080 + i, device="cuda")
    out, lse = sa.prefill(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q, w.cu_seqlens_kv,
                          max(lens_q), w.scale, w.causal, num_splits=ns,
                          max_seqlen_kv=max(lens_kv), rope=sa.RopeParams(**params))
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(k - q, k) for q, k in zip(lens_q, lens_kv)])
    qr = oracle.bf16_round(oracle.apply_rope(w.q, pos[:, None], **params))
    ro, rl = oracle.sink_attention(qr, w.k, w.v, w.sinks, w.cu_seqlens_q.cpu(),
                                   w.cu_seqlens_kv.cpu(), w.scale, w.causal)
    slack = prefill_lse_slack(w.q, pos, params, w.k, w.cu_seqlens_q, w.cu_seqlens_kv, hq, hkv,
                              w.scale, w.causal)
    _compare(out, lse, ro, rl, f"prefill rope case {i}", slack)
