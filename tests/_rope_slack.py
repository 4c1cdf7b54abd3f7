"""Extra lse tolerance for attention on rotated queries.

The kernels rotate q in fp32 and round the result to bf16; the oracle rotates in fp64 and
rounds the same way.  Where the exact rotated value lies within the fp32 computation's
error of a bf16 rounding midpoint, the two can round to neighbouring bf16 values (one ulp
apart: within the rotation's own tolerance).  Such an element moves the scores of its
row: a score by at most scale * sum_i ulp_i * |k_ji| over the row's ambiguous elements i,
and the row's lse, a log-sum-exp of its scores, by at most the largest of those moves.
The functions below return that bound per row (0 for rows with no ambiguous element), to
be added to the usual lse tolerance.  The fp32 rotation m (a cos - b sin) of a pair (a, b)
is off by at most about m (|a| + |b|) 2^-22 (cos and sin to an fp32 ulp, each product and
the difference rounded once); EPS = 2^-20 takes four times that.
"""
import numpy as np

import oracle

EPS = 2.0 ** -20


def _ambiguous_ulps(r, q, params):
    """One bf16 ulp where the fp64 rotation r may round either way under the fp32 error
    bound, else 0.  q: the unrotated input (pair magnitudes)."""
    q = np.asarray(q.float().cpu().numpy() if hasattr(q, "cpu") else q, dtype=np.float64)
    d = q.shape[-1]
    pair = np.abs(q[..., : d // 2]) + np.abs(q[..., d // 2:])
    m = oracle.yarn_mscale(params["factor"]) if params["factor"] > 1 else 1.0
    e = m * np.concatenate([pair, pair], axis=-1) * EPS
    return np.abs(oracle.bf16_round(r + e) - oracle.bf16_round(r - e))


def _row_bound(u_rows, k_rows, scale, vis):
    """max over visible keys j of scale * sum_i u[row, i] |k[j, i]| ; vis [rows, keys]."""
    if not u_rows.any() or k_rows.shape[0] == 0:
        return np.zeros(u_rows.shape[0])
    s = scale * (u_rows @ np.abs(k_rows).T)
    s = np.where(vis, s, 0.0)
    return s.max(axis=1)


def prefill_lse_slack(q, positions, params, k, cu_q, cu_kv, hq, hkv, scale, causal):
    """q [T, Hq, D] (the unrotated bf16 input), positions [T] -> slack [T, Hq]."""
    r = oracle.apply_rope(q, np.asarray(positions)[:, None], **params)
    u = _ambiguous_ulps(r, q, params)
    k = np.asarray(k.float().cpu().numpy() if hasattr(k, "cpu") else k, dtype=np.float64)
    cq = np.asarray(cu_q.cpu() if hasattr(cu_q, "cpu") else cu_q, dtype=np.int64)
    ck = np.asarray(cu_kv.cpu() if hasattr(cu_kv, "cpu") else cu_kv, dtype=np.int64)
    out = np.zeros(u.shape[:2])
    grp = hq // hkv
    for b in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
        lq, lk = q1 - q0, k1 - k0
        i = np.arange(lq)[:, None]
        j = np.arange(lk)[None, :]
        vis = (j <= i + lk - lq) if causal else np.ones((lq, lk), bool)
        for h in range(hq):
            out[q0:q1, h] = _row_bound(u[q0:q1, h, :], k[h // grp, k0:k1, :], scale, vis)
    return out


def decode_lse_slack(q, lens_kv, params, k, cu_kv, hq, hkv, scale, causal):
    """q [B, q_len, Hq, D] rotated at Lk - q_len + t -> slack [B, q_len, Hq]."""
    b_, ql = q.shape[0], q.shape[1]
    lens = np.asarray(lens_kv)
    pos = (lens[:, None] - ql + np.arange(ql)[None, :])[:, :, None]
    r = oracle.apply_rope(q, pos, **params)
    u = _ambiguous_ulps(r, q, params)
    k = np.asarray(k.float().cpu().numpy() if hasattr(k, "cpu") else k, dtype=np.float64)
    ck = np.asarray(cu_kv.cpu() if hasattr(cu_kv, "cpu") else cu_kv, dtype=np.int64)
    out = np.zeros(u.shape[:3])
    grp = hq // hkv
    for b in range(b_):
        k0, k1 = ck[b], ck[b + 1]
        lk = k1 - k0
        t = np.arange(ql)[:, None]
        j = np.arange(lk)[None, :]
        vis = (j <= lk - ql + t) if causal else np.ones((ql, lk), bool)
        for h in range(hq):
            out[b, :, h] = _row_bound(u[b, :, h, :], k[h // grp, k0:k1, :], scale, vis)
    return out
