"""GPU parity of YaRN rotary embedding (fused into the attention Q loads and into the
paged KV append, and the standalone rotation) against the fp64 CPU oracle.

Tolerances: a rotated vector is rounded to bf16, so element-wise |gpu - ref| <=
2^-8 |ref| + 1e-4 (one bf16 ulp plus float cos/sin).  Rotated q and k are attention
inputs stored as bf16, so the oracle's attention takes the same rounding of its fp64
rotation (bf16_round) and the usual bounds apply (max-abs 2e-2, mean-abs 2e-3, lse
1e-3)."""
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
YARN = dict(theta=150000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0, beta_slow=1.0)
PLAIN = dict(theta=10000.0, factor=1.0, original_max_pos=4096, beta_fast=32.0, beta_slow=1.0)


def _say(msg):
    print(f"[rope] {msg}", flush=True)
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


def _compare(out, lse, ro, rl, what, lse_slack=None):
    o = _np(out).reshape(ro.shape)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ro)
    assert err.max() <= MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    l = _np(lse).reshape(rl.shape)
    assert np.array_equal(np.isneginf(l), np.isneginf(rl)), f"{what}: -inf lse pattern"
    fin = np.isfinite(rl)
    if fin.any():
        tol = LSE_TOL if lse_slack is None else LSE_TOL + np.asarray(lse_slack).reshape(rl.shape)[fin]
        assert np.all(np.abs(l[fin] - rl[fin]) <= tol), f"{what}: lse"


@pytest.mark.parametrize("params", [YARN, PLAIN], ids=["yarn", "plain"])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_apply_matches_oracle(sa, params, d):
    g = torch.Generator(device="cuda").manual_seed(800 + d)
    tokens, heads = 300, 3
    x = torch.randn(tokens, heads, d, generator=g, device="cuda").to(torch.bfloat16)
    pos = torch.randint(0, 131072, (tokens,), generator=g, device="cuda", dtype=torch.int32)
    pos[:4] = torch.tensor([0, 1, 4095, 131071], dtype=torch.int32)
    ref = oracle.apply_rope(x, pos.cpu()[:, None], **params)
    _say(f"rope_apply NHD d={d} factor={params['factor']}")
    y = x.clone()
    sa.rope_apply(y, pos, sa.RopeParams(**params))
    torch.cuda.synchronize()
    err = np.abs(_np(y) - ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-4), err.max()
    # the same rotation through an HND view [heads, tokens, D]
    xh = x.permute(1, 0, 2).contiguous()
    sa.rope_apply(xh, pos, sa.RopeParams(**params), token_dim=1, head_dim_axis=0)
    torch.cuda.synchronize()
    assert torch.equal(xh.permute(1, 0, 2), y)


def test_decode_with_rope(sa):
    """Decode rotates each query at its position Lk - q_len + t (keys as given)."""
    for ql, hq, hkv, d, ns in ((1, 64, 8, 64, 0), (4, 64, 4, 128, 0), (2, 32, 2, 64, 3)):
        w = wl.make_decode([7, 1500, 4100, 33], ql, hq, hkv, d, ("normal", 0, 2),
                           1 / math.sqrt(d), True, ns, seed=810 + ql, device="cuda")
        _say(f"decode rope q_len={ql} hq={hq} hkv={hkv} d={d}")
        out, lse = sa.decode(w.q, w.k, w.v, w.sinks, w.cu_seqlens_kv, w.max_kv, w.scale,
                             w.causal, ns, rope=sa.RopeParams(**YARN))
        torch.cuda.synchronize()
        lens = np.array(w.lens_kv)
        pos = (lens[:, None] - ql + np.arange(ql)[None, :])[:, :, None]   # [B, q_len, 1]
        qr = oracle.bf16_round(oracle.apply_rope(w.q, pos, **YARN))
        ro, rl = oracle.sink_attention_decode(qr, w.k, w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                              w.scale, w.causal)
        slack = decode_lse_slack(w.q, w.lens_kv, YARN, w.k, w.cu_seqlens_kv, hq, hkv, w.scale,
                                 w.causal)
        _compare(out, lse, ro, rl, f"decode rope q_len={ql}", slack)


def test_prefill_with_rope(sa):
    """Prefill rotates query i at position Lk - Lq + i (a cached prefix shifts it)."""
    lq, lk = [200, 37, 513], [900, 37, 513]
    w = wl.make_prefill(lq, lk, 16, 4, 128, ("normal", 0, 2), 1 / math.sqrt(128), True,
                        seed=820, device="cuda")
    _say("prefill rope")
    out, lse = sa.prefill(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q, w.cu_seqlens_kv, w.max_q,
                          w.scale, w.causal, rope=sa.RopeParams(**YARN))
    torch.cuda.synchronize()
    pos = np.concatenate([np.arange(a, b) for a, b in zip(np.array(lk) - np.array(lq), lk)])
    qr = oracle.bf16_round(oracle.apply_rope(w.q, pos[:, None], **YARN))
    ro, rl = oracle.sink_attention(qr, w.k, w.v, w.sinks, w.cu_seqlens_q.cpu(),
                                   w.cu_seqlens_kv.cpu(), w.scale, w.causal)
    slack = prefill_lse_slack(w.q, pos, YARN, w.k, w.cu_seqlens_q, w.cu_seqlens_kv, 16, 4,
                              w.scale, w.causal)
    _compare(out, lse, ro, rl, "prefill rope", slack)


def test_append_rope_then_paged_decode(sa):
    """One engine step with YaRN: keys rotated as they are appended to the paged cache,
    the query rotated as the decode kernel loads it."""
    ql, hq, hkv, d, ps = 1, 64, 8, 64, 16
    lens = [100, 2049, 5000, 17]
    w = wl.make_decode(lens, ql, hq, hkv, d, ("normal", 0, 2), 0.125, True, 0, seed=830,
                       device="cuda")
    # the whole KV goes in through the append (positions 0 .. L-1), rotated on the way
    pk = wl.make_paged(w, ps, seed=831, fill="nan")
    k_new = w.k.permute(1, 0, 2).contiguous()
    v_new = w.v.permute(1, 0, 2).contiguous()
    rope = sa.RopeParams(**YARN)
    _say("append with rope + paged decode with rope")
    sa.kv_append(k_new, v_new, w.cu_seqlens_kv, pk.kv_page_indptr, pk.kv_page_indices,
                 pk.kv_last_page_len, pk.k_cache, pk.v_cache, max(lens), rope=rope)
    out, lse = sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,
                               pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale,
                               w.causal, 0, rope=rope)
    torch.cuda.synchronize()
    kpos = np.concatenate([np.arange(lk) for lk in lens])
    kr = oracle.apply_rope(w.k, kpos[None, :], **YARN)                     # [Hkv, total, D]
    qpos = (np.array(lens)[:, None] - ql + np.arange(ql)[None, :])[:, :, None]
    qr = oracle.bf16_round(oracle.apply_rope(w.q, qpos, **YARN))
    ro, rl = oracle.sink_attention_decode(qr, oracle.bf16_round(kr), w.v, w.sinks, w.cu_seqlens_kv.cpu(),
                                          w.scale, w.causal)
    _compare(out, lse, ro, rl, "append+decode rope")
    # the cached keys themselves: one bf16 rounding of the oracle's rotation
    got, _ = oracle.gather_paged(pk.k_cache, pk.kv_page_indptr.cpu(), pk.kv_page_indices.cpu(),
                                 pk.kv_last_page_len.cpu(), ps)
    assert np.all(np.abs(got - kr) <= 2.0 ** -8 * np.abs(kr) + 1e-4)
