"""Runs the fp64 oracle over a large prefill on several CPU threads (test helper).

Query rows are independent, and query head h reads only KV head h // G, so the oracle's
``sink_attention`` is called unchanged on pieces (sequence, KV head, block of query rows)
with that KV head's query heads and the keys the block can see; the pieces are then put
back in place.  numpy releases the interpreter lock inside its array operations, so the
pieces run in parallel on a thread pool (no child processes: nothing is forked or
executed from a process that uses the GPU).  Inputs are plain float32 arrays (bf16
values are exact in float32).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def _piece(args):
    import oracle
    q, k, v, sinks, scale, causal = args
    n, nk = q.shape[0], k.shape[1]
    return oracle.sink_attention(q, k, v, sinks, [0, n], [0, nk], scale, causal)


def prefill_reference(q, k, v, sinks, cu_q, cu_kv, scale, causal, rows=256, workers=None):
    """fp64 (out [total_q, Hq, D], lse [total_q, Hq]) of the oracle for a packed prefill.

    q [total_q, Hq, D], k/v [Hkv, total_kv, D] as float32 numpy arrays (or anything the
    oracle accepts), sinks [Hq] float32 or None, cu_q/cu_kv host int sequences."""
    q = np.asarray(q, dtype=np.float32)
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    tq, hq, d = q.shape
    hkv = k.shape[0]
    g = hq // hkv
    sk = None if sinks is None else np.asarray(sinks, dtype=np.float32)
    tasks, where = [], []
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_kv[b]), int(cu_kv[b + 1])
        lq, lk = q1 - q0, k1 - k0
        for r0 in range(0, lq, rows):
            r1 = min(lq, r0 + rows)
            # rows [r0, r1) see keys j <= i + lk - lq, at most the first r1 + lk - lq; with
            # exactly that many keys the piece's own bottom-right alignment is the
            # sequence's: query i' = i - r0 sees j <= i' + nk - (r1 - r0)
            nk = max(0, min(lk, r1 + lk - lq)) if causal else lk
            for h in range(hkv):
                hs = slice(h * g, (h + 1) * g)
                tasks.append((q[q0 + r0:q0 + r1, hs], k[h:h + 1, k0:k0 + nk],
                              v[h:h + 1, k0:k0 + nk], None if sk is None else sk[hs],
                              scale, causal))
                where.append((q0 + r0, q0 + r1, hs))
    out = np.zeros((tq, hq, d))
    lse = np.full((tq, hq), -np.inf)
    n = workers or min(8, max(1, len(os.sched_getaffinity(0)) // 2))
    try:  # a few BLAS threads per piece, so the pieces themselves run side by side
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=2)
    except Exception:
        limit = None
    try:
        with ThreadPoolExecutor(max_workers=n) as pool:
            for (a, b_, hs), (o, l) in zip(where, pool.map(_piece, tasks)):
                out[a:b_, hs] = o
                lse[a:b_, hs] = l
    finally:
        if limit is not None:
            limit.unregister()
    return out, lse
