"""Stream decode plan: each KV head's token axis (all sequences back to back) cut into
equal ranges, one wavefront each, partials merged with the sinks.

CPU tests check the host plan; GPU tests check the partials slot by slot against the
oracle's chunk form (chunk bounds at the range cuts, no sink in any chunk), the merge
step alone, and the whole decode against the plain definition on ragged batches with
short and empty sequences and tokens outside every sequence.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from gqa_attention_sink_amd import sink_attn as sa_mod
from gqa_attention_sink_amd import workloads as wl

MAX_ABS, MEAN_ABS, LSE_TOL = 2e-2, 2e-3, 1e-3


def _say(msg):
    print(f"[stream] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(sa_mod.LIB_PATH):
        from gqa_attention_sink_amd.build import build
        build()
    return sa_mod.load()


# ---------------------------------------------------------------- host plan (no GPU)

@pytest.mark.parametrize("b,ql,hq,hkv,d,total,maxkv", [
    (64, 1, 64, 8, 64, 294802, 8192),     # gpt-oss-like batch
    (1, 1, 64, 8, 64, 32768, 32768),      # one long sequence
    (300, 2, 16, 4, 128, 3000, 1100),     # many short sequences
    (7, 4, 16, 4, 64, 20000, 5000),
    (3, 1, 8, 1, 64, 2000, 1500),
    (256, 4, 64, 4, 128, 256 * 32768, 32768),   # speculative decode: 64 rows, 4 waves
    (9, 2, 32, 2, 64, 30000, 9000),              # 32 rows, 2 waves
])
def test_stream_plan_properties(lib, b, ql, hq, hkv, d, total, maxkv):
    plan = sa_mod.decode_stream_plan(b, ql, hq, hkv, d, total, maxkv)
    assert plan is not None
    r, nph, s = plan
    assert r % 32 == 0 and r >= 32
    assert nph * r >= total                      # every token is in some range
    assert r >= math.ceil(maxkv / 16)            # a sequence overlaps at most 17 ranges
    assert s == min(17, math.ceil(maxkv / r) + 1)
    # any sequence of length <= maxkv starting anywhere overlaps at most s ranges
    for start in (0, 1, r - 1, r, 5 * r + 17):
        n = (start + maxkv - 1) // r - start // r + 1
        assert n <= s
    # the workspace of decode covers the stream layout
    rows = b * ql * hq
    need = (rows * s * d * 4 + 255) // 256 * 256 + rows * s * 4
    assert sa_mod.decode_workspace_bytes(b, ql, hq, hkv, d, maxkv, 0) >= need


@pytest.mark.parametrize("b,ql,hq,hkv,d,total,maxkv", [
    (4, 4, 64, 2, 64, 8000, 2000),    # 128 rows per KV head: chunk plan
    (4, 1, 64, 8, 64, 4000, 1024),    # one slot: the chunk kernel writes the result
])
def test_stream_plan_not_used(lib, b, ql, hq, hkv, d, total, maxkv):
    assert sa_mod.decode_stream_plan(b, ql, hq, hkv, d, total, maxkv) is None


def test_stream_partial_rejects(lib):
    fake = sa_mod.ctypes.c_void_p(0x1000)
    # workspace missing / too small / misaligned
    args = [fake, fake, fake, fake, 4, 1, 8000, 2000, 64, 8, 64, 0.1, 1]
    assert lib.sink_attn_decode_stream_partial(*args, None, 0, None, None) == 3
    assert lib.sink_attn_decode_stream_partial(*args, fake, 16, None, None) == 3
    need = sa_mod.decode_workspace_bytes(4, 1, 64, 8, 64, 2000, 0)
    assert lib.sink_attn_decode_stream_partial(*args, sa_mod.ctypes.c_void_p(0x1010), need,
                                               None, None) == 3
    # 128 rows per KV head: the stream plan does not apply (rejected before any launch)
    args2 = [fake, fake, fake, fake, 4, 2, 8000, 2000, 64, 1, 64, 0.1, 1]
    assert lib.sink_attn_decode_stream_partial(*args2, fake, 1 << 30, None, None) == 2
    # merge: missing output
    assert lib.sink_attn_decode_stream_merge(None, fake, 4, 1, 8000, 2000, 64, 8, 64, fake,
                                             1 << 30, None, None, None) == 1


# ---------------------------------------------------------------- GPU parity

def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def sa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sink_amd as pkg
    pkg.load()
    return pkg


def _compare(out, lse, ref_out, ref_lse, what):
    o = _np(out).reshape(ref_out.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ref_out)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    l = _np(lse).reshape(ref_lse.shape)
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_lse)), f"{what}: -inf lse pattern"
    fin = np.isfinite(ref_lse)
    if fin.any():
        assert np.abs(l[fin] - ref_lse[fin]).max() <= LSE_TOL, f"{what}: lse"


def _gapped(w, lead, tail):
    """The workload's K/V with `lead` tokens before the first sequence and `tail` after
    the last (NaN: no sequence may read them, not even times a zero probability) and
    kv_indptr shifted by `lead`."""
    hkv, tk, d = w.k.shape
    pre = torch.full((hkv, lead, d), float("nan"), dtype=torch.bfloat16, device=w.k.device)
    post = torch.full((hkv, tail, d), float("nan"), dtype=torch.bfloat16, device=w.k.device)
    k = torch.cat([pre, w.k, post], dim=1).contiguous()
    v = torch.cat([pre, w.v, post], dim=1).contiguous()
    ind = (w.cu_seqlens_kv + lead).to(torch.int32)
    return k, v, ind


STREAM_CASES = [
    # lens, q_len, hq, hkv, d, sink, causal
    ([1100, 5, 31, 32, 33, 0, 64, 100, 3, 700, 1, 2, 1500], 1, 64, 8, 64, ("normal", 0, 2), True),
    ([2000, 17, 0, 0, 90, 1, 1200], 3, 16, 4, 64, ("alt_neginf", 2, 1), True),
    ([50] * 40 + [1300], 2, 16, 2, 128, ("normal", 0, 2), True),
    ([4096, 2500, 1025], 4, 16, 4, 128, None, True),
    ([1500, 800, 3000], 1, 8, 1, 64, ("normal", 0, 2), False),
    # more than 16 rows per KV head: one workgroup of 2 or 4 wavefronts per range
    ([3000, 40, 1, 1200, 0, 5000], 4, 64, 4, 128, ("normal", 0, 2), True),      # 64 rows
    ([700, 33, 2100, 64, 5], 2, 32, 2, 64, ("alt_neginf", 2, 1), True),         # 32 rows
    ([1800, 90, 2600], 3, 32, 2, 128, ("normal", 0, 2), True),                  # 48 rows
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(STREAM_CASES)))
def test_stream_partials_match_oracle_chunks(sa, case):
    lens, ql, hq, hkv, d, sink, causal = STREAM_CASES[case]
    w = wl.make_decode(lens, ql, hq, hkv, d, sink, 1 / math.sqrt(d), causal, 0, seed=700 + case,
                       device="cuda")
    tk = w.k.shape[1]
    plan = sa.decode_stream_plan(len(lens), ql, hq, hkv, d, tk, w.max_kv)
    assert plan is not None, "the stream plan must apply to this case"
    r, nph, s = plan
    _say(f"partials case {case}: lens={lens} q_len={ql} hq={hq} hkv={hkv} d={d} R={r} S={s}")
    po, pl, _ = sa.decode_stream_partial(w.q, w.k, w.v, w.cu_seqlens_kv, w.max_kv, w.scale,
                                         causal)
    torch.cuda.synchronize()
    ind = w.cu_seqlens_kv.cpu().tolist()
    bounds, nslots = [], []
    for b in range(len(lens)):
        s0, e0 = ind[b], ind[b + 1]
        lk = e0 - s0
        first = s0 // r
        n = ((e0 - 1) // r - first + 1) if lk > 0 else 0
        nslots.append(n)
        bd = [0] + [min(lk, max(0, (first + c) * r - s0)) for c in range(1, s)] + [lk]
        bounds.append(bd)
    cu_q = torch.arange(len(lens) + 1, dtype=torch.int32) * ql
    q2 = w.q.reshape(-1, hq, d)
    _, _, ref_po, ref_pl = oracle.sink_attention_chunked(q2, w.k, w.v, w.sinks, cu_q,
                                                         w.cu_seqlens_kv.cpu(), w.scale, causal,
                                                         bounds, sink_chunks="none",
                                                         return_partials=True)
    ref_pl = ref_pl.reshape(len(lens), ql * hq, s)
    ref_po = ref_po.reshape(len(lens), ql * hq, s, d)
    gl = _np(pl).reshape(len(lens), ql * hq, s)
    go = _np(po).reshape(len(lens), ql * hq, s, d)
    for b in range(len(lens)):
        n = nslots[b]
        if n == 0:
            continue
        rl, ll = ref_pl[b, :, :n], gl[b, :, :n]
        assert np.array_equal(np.isneginf(ll), np.isneginf(rl)), f"seq {b}: empty-slot pattern"
        fin = np.isfinite(rl)
        if fin.any():
            assert np.abs(ll[fin] - rl[fin]).max() <= LSE_TOL, f"seq {b}: lse"
            err = np.abs(go[b, :, :n][fin] - ref_po[b, :, :n][fin])
            assert err.max() <= 1e-2 and err.mean() <= 1e-3, f"seq {b}: partial output"


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(STREAM_CASES)))
def test_stream_decode_matches_oracle(sa, case):
    lens, ql, hq, hkv, d, sink, causal = STREAM_CASES[case]
    w = wl.make_decode(lens, ql, hq, hkv, d, sink, 1 / math.sqrt(d), causal, 0, seed=720 + case,
                       device="cuda")
    _say(f"decode case {case}")
    out, lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, causal, 0)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, causal)
    _compare(out, lse, ro, rl, f"stream decode case {case}")
    # empty sequences: zero output, lse = sink (or -inf)
    for b, lk in enumerate(lens):
        if lk == 0:
            assert float(out[b].abs().max()) == 0.0


@pytest.mark.gpu
def test_stream_ignores_tokens_outside_sequences(sa):
    """kv_indptr starting after token 0 and ending before the last token: ranges cover
    those tokens too (NaN here), and no sequence may read them."""
    lens = [1200, 7, 300, 64]
    w = wl.make_decode(lens, 2, 16, 4, 64, ("normal", 0, 2), 0.125, True, 0, seed=740,
                       device="cuda")
    k, v, ind = _gapped(w, 45, 77)
    _say("gapped kv_indptr")
    assert sa.decode_stream_plan(len(lens), 2, 16, 4, 64, k.shape[1], w.max_kv) is not None
    out, lse = sa.decode(w.q, k, v, w.sinks, ind, w.max_kv, w.scale, True, 0)
    torch.cuda.synchronize()
    ro, rl = oracle.sink_attention_decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, True)
    _compare(out, lse, ro, rl, "gapped")


@pytest.mark.gpu
def test_stream_merge_step_equals_decode(sa):
    lens = [1100, 5, 2000, 0, 333]
    w = wl.make_decode(lens, 1, 64, 8, 64, ("normal", 0, 2), 0.125, True, 0, seed=750,
                       device="cuda")
    tk = w.k.shape[1]
    _say("partial + merge vs decode")
    out, lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, True, 0)
    _, _, ws = sa.decode_stream_partial(w.q, w.k, w.v, w.cu_seqlens_kv, w.max_kv, w.scale, True)
    o2, l2 = sa.decode_stream_merge(w.sinks, w.cu_seqlens_kv, tuple(w.q.shape), tk, 8, w.max_kv,
                                    ws)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    # the empty sequence: zero output and lse = its heads' sinks
    assert float(o2[3].abs().max()) == 0.0
    assert torch.allclose(l2[3, 0].float(), w.sinks.float(), atol=0, rtol=0)


@pytest.mark.gpu
def test_stream_decode_with_rope(sa):
    lens = [1500, 40, 700]
    w = wl.make_decode(lens, 2, 16, 4, 64, ("normal", 0, 2), 0.125, True, 0, seed=760,
                       device="cuda")
    rope = dict(theta=150000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0,
                beta_slow=1.0)
    _say("stream decode with YaRN rotation of q")
    out, lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale, True, 0,
                         rope=sa.RopeParams(**rope))
    torch.cuda.synchronize()
    # oracle: rotate each query row at its position Lk - q_len + t, rounded to bf16
    qr = np.zeros(tuple(w.q.shape))
    qn = _np(w.q)
    for b, lk in enumerate(lens):
        pos = np.array([lk - 2 + t for t in range(2)])[:, None] * np.ones((1, 16))
        qr[b] = oracle.bf16_round(oracle.apply_rope(qn[b], pos, **rope))
    ro, rl = oracle.sink_attention_decode(qr, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, True)
    _compare(out, lse, ro, rl, "stream rope")
