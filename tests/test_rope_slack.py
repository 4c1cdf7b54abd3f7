"""CPU pins of the rotated-attention lse slack (tests/_rope_slack.py).

An fp32 evaluation of the rotation, in the order a kernel takes it (angle formed and
reduced modulo 2 pi in double, cos and sin in float, m (a cos - b sin) in float), is
rounded to bf16 and compared with the oracle's fp64 rotation rounded the same way:
  * every element where the two roundings differ is one the slack marks ambiguous;
  * few elements are marked (the slack is not a blanket allowance);
  * the oracle's lse on the two rounded inputs differs by no more than the slack.
"""
import math

import numpy as np
import pytest

import oracle
from _rope_slack import _ambiguous_ulps, decode_lse_slack, prefill_lse_slack

YARN = dict(theta=150000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0, beta_slow=1.0)
PLAIN = dict(theta=10000.0, factor=1.0, original_max_pos=4096, beta_fast=32.0, beta_slow=1.0)


def _rotate_fp32(x, positions, params):
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    f = oracle.yarn_inv_freq(d, params["theta"], params["factor"], params["original_max_pos"],
                             params["beta_fast"], params["beta_slow"])
    ang = np.asarray(positions, dtype=np.float64)[..., None] * f
    red = ang - np.rint(ang / (2 * math.pi)) * (2 * math.pi)
    rf = red.astype(np.float32)
    c, s = np.cos(rf).astype(np.float32), np.sin(rf).astype(np.float32)
    m = np.float32(oracle.yarn_mscale(params["factor"]))
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([m * (a * c - b * s), m * (b * c + a * s)], axis=-1).astype(np.float64)


def _inputs(seed, t, h, d):
    r = np.random.default_rng(seed)
    q = oracle.bf16_round(r.standard_normal((t, h, d)))
    pos = r.integers(0, 131072, t)
    return q, pos


@pytest.mark.parametrize("params", [YARN, PLAIN], ids=["yarn", "plain"])
@pytest.mark.parametrize("d", [64, 128])
def test_flips_only_where_marked(params, d):
    q, pos = _inputs(7 + d, 3000, 4, d)
    ref = oracle.bf16_round(oracle.apply_rope(q, pos[:, None], **params))
    f32 = oracle.bf16_round(_rotate_fp32(q, pos[:, None], params))
    u = _ambiguous_ulps(oracle.apply_rope(q, pos[:, None], **params), q, params)
    flips = f32 != ref
    assert flips.sum() > 0                 # the effect is real at this size
    assert np.all(u[flips] > 0)            # and always inside the marked set
    assert np.all(np.abs(f32 - ref)[flips] <= u[flips])
    assert (u > 0).mean() < 1e-2           # the marked set stays small (under 1 %)


def test_prefill_lse_within_slack():
    rng = np.random.default_rng(11)
    lq, lk, hq, hkv, d = [300, 77], [700, 77], 8, 2, 64
    cq, ck = np.cumsum([0] + lq), np.cumsum([0] + lk)
    q = oracle.bf16_round(rng.standard_normal((cq[-1], hq, d)))
    k = oracle.bf16_round(rng.standard_normal((hkv, ck[-1], d)))
    v = oracle.bf16_round(rng.standard_normal((hkv, ck[-1], d)))
    pos = np.concatenate([np.arange(b - a, b) for a, b in zip(lq, lk)])
    scale = 1 / 8
    ref = oracle.bf16_round(oracle.apply_rope(q, pos[:, None], **YARN))
    f32 = oracle.bf16_round(_rotate_fp32(q, pos[:, None], YARN))
    _, l1 = oracle.sink_attention(ref, k, v, None, cq, ck, scale, True)
    _, l2 = oracle.sink_attention(f32, k, v, None, cq, ck, scale, True)
    slack = prefill_lse_slack(q, pos, YARN, k, cq, ck, hq, hkv, scale, True)
    fin = np.isfinite(l1)
    assert np.all(np.abs(l1[fin] - l2[fin]) <= slack[fin] + 1e-9)
    assert slack.max() > 0 and (slack > 0).mean() < 0.2


def test_decode_lse_within_slack():
    rng = np.random.default_rng(12)
    lens, ql, hq, hkv, d = [900, 1, 2500, 64], 4, 16, 2, 128
    ck = np.cumsum([0] + lens)
    q = oracle.bf16_round(rng.standard_normal((len(lens), ql, hq, d)))
    k = oracle.bf16_round(rng.standard_normal((hkv, ck[-1], d)))
    v = oracle.bf16_round(rng.standard_normal((hkv, ck[-1], d)))
    pos = (np.array(lens)[:, None] - ql + np.arange(ql)[None, :])[:, :, None]
    scale = 1 / math.sqrt(d)
    ref = oracle.bf16_round(oracle.apply_rope(q, pos, **YARN))
    f32 = oracle.bf16_round(_rotate_fp32(q, pos, YARN))
    _, l1 = oracle.sink_attention_decode(ref, k, v, None, ck, scale, True)
    _, l2 = oracle.sink_attention_decode(f32, k, v, None, ck, scale, True)
    slack = decode_lse_slack(q, lens, YARN, k, ck, hq, hkv, scale, True)
    fin = np.isfinite(l1)
    assert np.all(np.abs(l1[fin] - l2[fin]) <= slack.reshape(l1.shape)[fin] + 1e-9)
