"""Arbitrary-precision brute force of sink attention, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see ``oracle/sink_attention.py``).  Pure-Python loops over
every (token, head, key) with mpmath at a chosen number of decimal digits.  It takes
the definition from "GPT-OSS on day 0", section "Kernels for GPT-OSS" > "Sink
attention" literally, without the max subtraction: the softmax over the row's visible
scores plus one sink logit, the sink having no value row.  Used to check the float64
oracle's own rounding on inputs whose exact answer it can compute.
"""
from __future__ import annotations

import mpmath


def sink_attention_mp(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, sm_scale,
                      causal=True, dps=50):
    """q: nested lists [total_q][Hq][D]; k, v: [Hkv][total_kv][D]; sinks [Hq] (floats,
    may be -inf) or None.  Returns (out, lse) as nested lists of mpf."""
    with mpmath.workdps(dps):
        hq = len(q[0])
        hkv = len(k)
        gsz = hq // hkv
        d = len(q[0][0])
        scale = mpmath.mpf(sm_scale)
        out = []
        lse = []
        for b in range(len(cu_seqlens_q) - 1):
            q0, q1 = cu_seqlens_q[b], cu_seqlens_q[b + 1]
            k0, k1 = cu_seqlens_kv[b], cu_seqlens_kv[b + 1]
            lq, lk = q1 - q0, k1 - k0
            for i in range(lq):
                orow, lrow = [], []
                for h in range(hq):
                    g = h // gsz
                    sig = None if sinks is None else sinks[h]
                    terms = []          # (weight, value row or None for the sink)
                    if sig is not None and sig != float("-inf"):
                        terms.append((mpmath.exp(mpmath.mpf(sig)), None))
                    for j in range(lk):
                        if causal and j > i + lk - lq:
                            continue
                        s = scale * mpmath.fsum(mpmath.mpf(q[q0 + i][h][t]) *
                                                mpmath.mpf(k[g][k0 + j][t])
                                                for t in range(d))
                        terms.append((mpmath.exp(s), v[g][k0 + j]))
                    z = mpmath.fsum(w for w, _ in terms)
                    if z == 0:
                        orow.append([mpmath.mpf(0)] * d)
                        lrow.append(mpmath.mpf("-inf"))
                        continue
                    o = [mpmath.fsum(w * mpmath.mpf(row[t]) for w, row in terms
                                     if row is not None) / z for t in range(d)]
                    orow.append(o)
                    lrow.append(mpmath.log(z))
                out.append(orow)
                lse.append(lrow)
        return out, lse
