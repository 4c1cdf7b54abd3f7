"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Definition: "GPT-OSS on day 0", section "Kernels for GPT-OSS" > "Sink attention"
(formula, max-subtracted online softmax, sink as the initial running maximum, sink in
the first KV block only).  The pages print no numeric example, so every pin is a hand
derivation, a closed form, an invariant, a library routine on a special case, or an
arbitrary-precision brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (flops_causal, merge_partials, sink_attention, sink_attention_chunked,
                    sink_attention_decode)
from oracle.bruteforce import sink_attention_mp

HERE = os.path.dirname(os.path.abspath(__file__))
pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand_case(rng, lens_q, lens_kv, hq, hkv, d, sink_std=2.0, neg_heads=()):
    tq, tk = sum(lens_q), sum(lens_kv)
    q = rng.standard_normal((tq, hq, d))
    k = rng.standard_normal((hkv, tk, d))
    v = rng.standard_normal((hkv, tk, d))
    s = rng.standard_normal(hq) * sink_std
    for h in neg_heads:
        s[h] = -np.inf
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum(lens_kv)]).astype(np.int64)
    return q, k, v, s, cq, ck


def _logistic(x):
    return 1.0 / (1.0 + math.exp(-x))


# ---------------------------------------------------------------- golden fixtures
def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "ln": math.log}))


def test_golden_closed_forms():
    """Hand-derived worked cases (tests/golden/closed_forms.json)."""
    data = json.load(open(os.path.join(HERE, "golden", "closed_forms.json")))
    for case in data["cases"]:
        sinks = [float(x) for x in case["sinks"]]
        out, lse = sink_attention(np.array(case["q"], float), np.array(case["k"], float),
                                  np.array(case["v"], float), np.array(sinks),
                                  case["cu_q"], case["cu_kv"], case["sm_scale"],
                                  case["causal"])
        exp_out = np.vectorize(_ev)(np.array(case["out"], dtype=object)).astype(float)
        exp_lse = np.vectorize(_ev)(np.array(case["lse"], dtype=object)).astype(float)
        np.testing.assert_allclose(out, exp_out, rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(lse, exp_lse, rtol=0, atol=1e-14, err_msg=case["name"])


# ---------------------------------------------------------------- P2 single key
@pytest.mark.parametrize("seed", range(5))
def test_single_key_closed_form(seed):
    """out = v * logistic(s - sink), lse = logaddexp(s, sink), for any scale."""
    rng = np.random.default_rng(seed)
    d, hq = 8, 3
    q, k, v, s, cq, ck = _rand_case(rng, [1], [1], hq, 1, d, sink_std=3.0)
    scale = 0.37
    out, lse = sink_attention(q, k, v, s, cq, ck, scale, True)
    for h in range(hq):
        sc = scale * float(np.dot(q[0, h], k[0, 0]))
        np.testing.assert_allclose(out[0, h], v[0, 0] * _logistic(sc - s[h]), rtol=1e-13, atol=1e-15)
        assert abs(lse[0, h] - np.logaddexp(sc, s[h])) < 1e-13


# ---------------------------------------------------------------- P3 equal scores
def test_equal_scores_closed_form():
    """All keys equal (so every score is s): out = logistic(s + ln n - sink) * mean(v)."""
    rng = np.random.default_rng(1)
    n, d, hq = 37, 16, 2
    q = rng.standard_normal((1, hq, d))
    krow = rng.standard_normal(d)
    k = np.tile(krow, (1, n, 1))
    v = rng.standard_normal((1, n, d))
    sinks = np.array([0.3, -1.7])
    out, lse = sink_attention(q, k, v, sinks, [0, 1], [0, n], 0.25, False)
    for h in range(hq):
        s = 0.25 * float(q[0, h] @ krow)
        w = _logistic(s + math.log(n) - sinks[h])
        np.testing.assert_allclose(out[0, h], w * v[0].mean(axis=0), rtol=1e-12, atol=1e-14)
        assert abs(lse[0, h] - np.logaddexp(s + math.log(n), sinks[h])) < 1e-12


# ---------------------------------------------------------------- P4 sink -inf == SDPA
@pytest.mark.parametrize("lq,lk", [(7, 7), (3, 11), (1, 9), (16, 16)])
def test_neg_inf_sink_matches_sdpa(lq, lk):
    """With every sink -inf the method is ordinary attention: compare with torch's
    scaled_dot_product_attention in fp64 with an explicit bottom-right mask."""
    rng = np.random.default_rng(lq * 100 + lk)
    hq, hkv, d = 6, 2, 8
    q, k, v, s, cq, ck = _rand_case(rng, [lq], [lk], hq, hkv, d)
    s[:] = -np.inf
    out, lse = sink_attention(q, k, v, s, cq, ck, 0.3, True)
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                         # [Hq, Lq, D]
    kt = torch.from_numpy(k).repeat_interleave(g, dim=0)             # [Hq, Lk, D]
    vt = torch.from_numpy(v).repeat_interleave(g, dim=0)
    i = torch.arange(lq)[:, None]
    j = torch.arange(lk)[None, :]
    mask = j <= i + (lk - lq)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.3)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)
    sc = torch.einsum("hid,hjd->hij", qt, kt) * 0.3
    ref_lse = torch.logsumexp(sc.masked_fill(~mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(lse, ref_lse.T.numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P5 mass identity
def test_mass_identity_v_ones():
    """With V == 1 every row's output is the key mass: out = 1 - e^(sink - lse)."""
    rng = np.random.default_rng(5)
    q, k, v, s, cq, ck = _rand_case(rng, [5, 9], [12, 9], 8, 2, 16, neg_heads=(3,))
    v[:] = 1.0
    out, lse = sink_attention(q, k, v, s, cq, ck, 0.25, True)
    expect = 1.0 - np.exp(s[None, :] - lse)
    np.testing.assert_allclose(out, np.repeat(expect[:, :, None], 16, axis=2), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P6 limits
def test_sink_limits():
    rng = np.random.default_rng(6)
    q, k, v, s, cq, ck = _rand_case(rng, [4], [4], 2, 1, 8)
    s[:] = 700.0                                     # sink dominates every key
    out, lse = sink_attention(q, k, v, s, cq, ck, 0.2, True)
    assert np.abs(out).max() < 1e-250
    np.testing.assert_allclose(lse, 700.0, rtol=0, atol=1e-12)
    # sink equal to the only score: half the mass each
    q, k, v, s, cq, ck = _rand_case(rng, [1], [1], 2, 1, 8)
    sc = 0.2 * (q[0] @ k[0, 0])
    out, lse = sink_attention(q, k, v, sc, cq, ck, 0.2, True)
    np.testing.assert_allclose(out[0], np.tile(v[0, 0] / 2, (2, 1)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse[0], sc + math.log(2), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- P1 + P7 split/merge
def _random_bounds(rng, lk, n):
    cuts = sorted(int(x) for x in rng.integers(0, lk + 1, size=n - 1))
    return [0] + cuts + [lk]


@pytest.mark.parametrize("seed", range(4))
def test_split_invariance(seed):
    """Every partition of the keys (empty chunks, size-1 chunks, many chunks) merges to
    the unsplit result when the sink joins the first chunk only."""
    rng = np.random.default_rng(seed)
    lens_kv = [1, 33, 70, 5]
    lens_q = [1, 4, 4, 2]
    q, k, v, s, cq, ck = _rand_case(rng, lens_q, lens_kv, 8, 2, 16, neg_heads=(0, 5))
    ref_o, ref_l = sink_attention(q, k, v, s, cq, ck, 0.25, True)
    for n in (1, 2, 5, 32):
        bounds = [_random_bounds(rng, lk, n) for lk in lens_kv]
        o, l = sink_attention_chunked(q, k, v, s, cq, ck, 0.25, True, bounds)
        np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l, ref_l, rtol=1e-12, atol=1e-13)


def test_split_negative_controls():
    """Putting the sink in every chunk, or in none, changes the answer."""
    rng = np.random.default_rng(11)
    q, k, v, s, cq, ck = _rand_case(rng, [2], [64], 4, 1, 16)
    bounds = [[0, 16, 32, 48, 64]]
    ref_o, ref_l = sink_attention(q, k, v, s, cq, ck, 0.25, True)
    for mode in ("all", "none"):
        o, l = sink_attention_chunked(q, k, v, s, cq, ck, 0.25, True, bounds, sink_chunks=mode)
        assert np.abs(l - ref_l).max() > 1e-3, mode


def test_merge_handles_empty_chunks():
    po = np.zeros((3, 4, 2))
    po[0, 1] = [1.0, 2.0]
    po[1, 0] = [3.0, -1.0]
    po[1, 2] = [5.0, 1.0]
    pl = np.full((3, 4), -np.inf)
    pl[0, 1] = 0.5
    pl[1, 0] = 0.0
    pl[1, 2] = math.log(3.0)
    out, lse = merge_partials(po, pl)
    np.testing.assert_allclose(out[0], [1.0, 2.0])
    assert abs(lse[0] - 0.5) < 1e-15
    np.testing.assert_allclose(out[1], [(3.0 + 3 * 5.0) / 4, (-1.0 + 3 * 1.0) / 4])
    assert abs(lse[1] - math.log(4.0)) < 1e-15
    assert np.all(out[2] == 0) and np.isneginf(lse[2])


# ---------------------------------------------------------------- P8 GQA == MHA
def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(8)
    hq, hkv = 12, 3
    q, k, v, s, cq, ck = _rand_case(rng, [6, 3], [6, 10], hq, hkv, 8)
    o1, l1 = sink_attention(q, k, v, s, cq, ck, 0.3, True)
    g = hq // hkv
    o2, l2 = sink_attention(q, np.repeat(k, g, axis=0), np.repeat(v, g, axis=0), s, cq, ck, 0.3, True)
    np.testing.assert_allclose(o1, o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- P9 brute force
@pytest.mark.parametrize("seed", range(3))
def test_bruteforce_mpmath(seed):
    """50-digit brute force on tiny integer inputs with a power-of-two scale."""
    rng = np.random.default_rng(seed)
    hq, hkv, d = 4, 2, 4
    lens_q, lens_kv = [2, 1], [3, 4]
    tq, tk = sum(lens_q), sum(lens_kv)
    q = rng.integers(-3, 4, (tq, hq, d)).astype(float)
    k = rng.integers(-3, 4, (hkv, tk, d)).astype(float)
    v = rng.integers(-3, 4, (hkv, tk, d)).astype(float)
    sinks = [0.5, float("-inf"), -1.25, 2.0]
    cq, ck = [0, 2, 3], [0, 3, 7]
    out, lse = sink_attention(q, k, v, np.array(sinks), cq, ck, 0.5, True)
    mo, ml = sink_attention_mp(q.tolist(), k.tolist(), v.tolist(), sinks, cq, ck, 0.5, True)
    np.testing.assert_allclose(out, np.array(mo, dtype=float), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.array(ml, dtype=float), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P10 causal/offset
def test_masked_positions_do_not_matter():
    rng = np.random.default_rng(10)
    lq, lk = 5, 9
    q, k, v, s, cq, ck = _rand_case(rng, [lq], [lk], 4, 2, 8)
    o1, l1 = sink_attention(q, k, v, s, cq, ck, 0.3, True)
    k2, v2 = k.copy(), v.copy()
    # key lk-1 is visible only to the last query; rows < lq-1 must not see it
    k2[:, lk - 1] = 1e3
    v2[:, lk - 1] = 1e3
    o2, l2 = sink_attention(q, k2, v2, s, cq, ck, 0.3, True)
    assert np.array_equal(o1[:lq - 1], o2[:lq - 1]) and np.array_equal(l1[:lq - 1], l2[:lq - 1])
    assert not np.allclose(o1[lq - 1], o2[lq - 1])


def test_packed_equals_alone():
    rng = np.random.default_rng(12)
    lens_q, lens_kv = [3, 6, 2], [7, 6, 12]
    q, k, v, s, cq, ck = _rand_case(rng, lens_q, lens_kv, 4, 1, 8)
    o, l = sink_attention(q, k, v, s, cq, ck, 0.3, True)
    for b in range(3):
        qs = q[cq[b]:cq[b + 1]]
        ks = k[:, ck[b]:ck[b + 1]]
        vs = v[:, ck[b]:ck[b + 1]]
        ob, lb = sink_attention(qs, ks, vs, s, [0, lens_q[b]], [0, lens_kv[b]], 0.3, True)
        assert np.array_equal(ob, o[cq[b]:cq[b + 1]]) and np.array_equal(lb, l[cq[b]:cq[b + 1]])


@pytest.mark.parametrize("lq,lk", [(4, 4), (3, 10)])
def test_spike_at_causal_limit(lq, lk):
    """A key with a huge score and a distinctive value placed exactly at query i's
    causal limit dominates row i; placed one past the limit it is invisible."""
    d = 8
    for i in range(lq):
        limit = i + lk - lq
        for pos, visible in ((limit, True), (limit + 1, False)):
            if pos >= lk:
                continue
            q = np.zeros((lq, 1, d)); q[i, 0, 0] = 1.0
            k = np.zeros((1, lk, d)); k[0, pos, 0] = 100.0
            v = np.zeros((1, lk, d)); v[0, pos, :] = 7.0
            out, _ = sink_attention(q, k, v, np.array([0.0]), [0, lq], [0, lk], 1.0, True)
            if visible:
                np.testing.assert_allclose(out[i, 0], 7.0, rtol=1e-12)
            else:
                assert np.abs(out[i, 0]).max() == 0.0


# ---------------------------------------------------------------- P11 permutation
def test_key_permutation_invariance_noncausal():
    rng = np.random.default_rng(13)
    q, k, v, s, cq, ck = _rand_case(rng, [5], [17], 4, 2, 8)
    o1, l1 = sink_attention(q, k, v, s, cq, ck, 0.3, False)
    perm = rng.permutation(17)
    o2, l2 = sink_attention(q, k[:, perm], v[:, perm], s, cq, ck, 0.3, False)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- degenerate
def test_empty_kv_rows():
    """A sequence with no keys: out 0, lse = sink (or -inf with no sink)."""
    q = np.ones((2, 2, 4))
    k = np.zeros((1, 0, 4)); v = np.zeros((1, 0, 4))
    out, lse = sink_attention(q, k, v, np.array([1.5, -np.inf]), [0, 2], [0, 0], 1.0, False)
    assert np.all(out == 0)
    np.testing.assert_array_equal(lse[:, 0], [1.5, 1.5])
    assert np.all(np.isneginf(lse[:, 1]))


def test_decode_layout_matches_prefill_layout():
    rng = np.random.default_rng(14)
    b, ql, hq, hkv, d = 3, 4, 8, 2, 16
    lens = [9, 4, 20]
    q = rng.standard_normal((b, ql, hq, d))
    k = rng.standard_normal((hkv, sum(lens), d))
    v = rng.standard_normal((hkv, sum(lens), d))
    s = rng.standard_normal(hq)
    ind = np.concatenate([[0], np.cumsum(lens)])
    o, l = sink_attention_decode(q, k, v, s, ind, 0.25, True)
    for bi in range(b):
        ob, lb = sink_attention(q[bi], k[:, ind[bi]:ind[bi + 1]], v[:, ind[bi]:ind[bi + 1]], s,
                                [0, ql], [0, lens[bi]], 0.25, True)
        assert np.array_equal(o[bi], ob) and np.array_equal(l[bi], lb)


def test_flops_causal_closed_form():
    assert flops_causal([0, 6000], [0, 6000], 64, 128) == 4 * 128 * 64 * (6000 * 6001 // 2)
    assert flops_causal([0, 4], [0, 10], 2, 8) == 4 * 8 * 2 * (7 + 8 + 9 + 10)
    assert flops_causal([0, 3], [0, 5], 1, 1, causal=False) == 4 * 15
