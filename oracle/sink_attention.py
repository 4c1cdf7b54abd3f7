"""fp64 CPU oracle for grouped-query attention with a learned per-head softmax sink.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may call it.  It shares no code with the HIP kernels or their host runtime.

What it computes, and where the definition comes from
-----------------------------------------------------
"GPT-OSS on day 0" (Perplexity), section "Kernels for GPT-OSS" > "Sink attention":
the attention of a head is ``softmax(q @ k^T * sm_scale + sink) * V``; the softmax is
evaluated with the running maximum subtracted; the running state starts from the
head's sink value; and when attention is split into blocks along the KV length the
sink is included in the first block only.  The same page's "model deltas" list says
every attention head owns one pre-trained sink parameter that takes part in the
softmax, and that attention is grouped-query (GQA).

Readings of points the pages leave open:

* The sink is one extra logit column with no value row.  Adding the same scalar to
  every logit would be a no-op under softmax, so the only reading that changes the
  result is: the sink term enters the denominator and contributes nothing to the
  numerator.
* The sink is not multiplied by ``sm_scale`` (operator precedence of the formula).
* One sink per query head; ``sinks is None`` means "no sink" (every sink = -inf).
* GQA head map: query head ``h`` reads KV head ``h // (Hq // Hkv)``.
* Causal alignment is bottom-right: query ``i`` of a sequence with ``Lq`` queries and
  ``Lk`` keys sees key ``j`` iff ``j <= i + Lk - Lq``.
* ``lse`` is the natural-log partition function including the sink term.
* A row that sees no key and has sink -inf has out = 0 and lse = -inf; a row that sees
  no key but has a finite sink has out = 0 and lse = sink.
* KV layout is HND, ``[kv_head, token, head_dim]`` with tokens contiguous per head
  ("Hosting Qwen on Blackwell", introduction: KV caches are stored head-major so they
  can be split or concatenated by head).

All arithmetic is float64 on the (exactly representable) bf16/fp32 input values.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "sink_attention",
    "sink_attention_decode",
    "sink_attention_chunked",
    "merge_partials",
    "flops_causal",
]

_QBLOCK = 512  # query rows per matrix product; limits temporary memory only


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16/fp16/fp32) or array to float64."""
    if hasattr(x, "detach"):  # torch tensor, imported lazily by the caller
        x = x.detach().cpu()
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def _visible(lq: int, lk: int, r0: int, r1: int, causal: bool) -> np.ndarray:
    """Boolean [r1-r0, lk]: key j visible to query i (bottom-right causal alignment)."""
    i = np.arange(r0, r1, dtype=np.int64)[:, None]
    j = np.arange(lk, dtype=np.int64)[None, :]
    vis = np.ones((r1 - r0, lk), dtype=bool)
    if causal:
        vis &= j <= i + (lk - lq)
    return vis


def _softmax_with_sink(s: np.ndarray, vis: np.ndarray, sig: np.ndarray, v: np.ndarray):
    """One softmax-with-sink over the last axis.

    s   [G, n, lk] scores (already scaled), vis [n, lk], sig [G] sink logits, v [lk, D].
    Returns out [G, n, D] and lse [G, n].

    Max-subtracted form ("Sink attention": softmax is computed with the maximum taken
    out):  M = max(sink, max_j s_j),  Z = e^(sink-M) + sum_j e^(s_j-M),
    out = sum_j e^(s_j-M) v_j / Z,  lse = M + ln Z.
    """
    g, n, lk = s.shape
    s = np.where(vis[None, :, :], s, -np.inf)
    smax = s.max(axis=-1) if lk > 0 else np.full((g, n), -np.inf)
    m = np.maximum(sig[:, None], smax)                      # [G, n]
    dead = np.isneginf(m)                                   # no key and no sink
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[..., None])                       # masked -> exp(-inf) = 0
    z = np.exp(sig[:, None] - m_safe) + e.sum(axis=-1)     # sink: denominator only
    num = e @ v                                             # [G, n, D]
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(dead[..., None], 0.0, num / np.where(dead, 1.0, z)[..., None])
        lse = np.where(dead, -np.inf, m_safe + np.log(np.where(dead, 1.0, z)))
    return out, lse


def sink_attention(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, sm_scale: float,
                   causal: bool = True):
    """Variable-length sink attention over packed queries and HND keys/values.

    q  [total_q, Hq, D]    (token-major, "NHD")
    k  [Hkv, total_kv, D]  (head-major, "HND");  v likewise
    sinks [Hq] or None;  cu_seqlens_q / cu_seqlens_kv [B+1] cumulative lengths.
    Returns (out [total_q, Hq, D], lse [total_q, Hq]) in float64.
    """
    q = _f64(q); k = _f64(k); v = _f64(v)
    cq = _i64(cu_seqlens_q); ck = _i64(cu_seqlens_kv)
    tq, hq, d = q.shape
    hkv = k.shape[0]
    assert hq % hkv == 0, "query heads must be a multiple of KV heads"
    gsz = hq // hkv
    sig_all = np.full(hq, -np.inf) if sinks is None else _f64(sinks).reshape(hq)
    out = np.zeros((tq, hq, d))
    lse = np.full((tq, hq), -np.inf)
    for b in range(len(cq) - 1):
        q0, q1 = int(cq[b]), int(cq[b + 1])
        k0, k1 = int(ck[b]), int(ck[b + 1])
        lq, lk = q1 - q0, k1 - k0
        for g in range(hkv):
            heads = slice(g * gsz, (g + 1) * gsz)           # GQA: heads sharing KV head g
            kb = k[g, k0:k1, :]
            vb = v[g, k0:k1, :]
            sig = sig_all[heads]
            for r0 in range(0, lq, _QBLOCK):
                r1 = min(lq, r0 + _QBLOCK)
                qb = np.transpose(q[q0 + r0:q0 + r1, heads, :], (1, 0, 2))   # [G, n, D]
                s = (qb @ kb.T) * sm_scale                  # sink is NOT scaled
                o, l = _softmax_with_sink(s, _visible(lq, lk, r0, r1, causal), sig, vb)
                out[q0 + r0:q0 + r1, heads, :] = np.transpose(o, (1, 0, 2))
                lse[q0 + r0:q0 + r1, heads] = l.T
    return out, lse


def sink_attention_decode(q, k, v, sinks, kv_indptr, sm_scale: float, causal: bool = True):
    """Decode layout: q [B, q_len, Hq, D]; KV of sequence b is tokens
    [kv_indptr[b], kv_indptr[b+1]) of the HND tensors and already holds the q_len new
    tokens, so query t sits at absolute position Lk - q_len + t.
    Returns (out [B, q_len, Hq, D], lse [B, q_len, Hq]) in float64."""
    q = _f64(q)
    bsz, ql, hq, d = q.shape
    cu_q = np.arange(bsz + 1, dtype=np.int64) * ql
    out, lse = sink_attention(q.reshape(bsz * ql, hq, d), k, v, sinks, cu_q,
                              kv_indptr, sm_scale, causal)
    return out.reshape(bsz, ql, hq, d), lse.reshape(bsz, ql, hq)


def merge_partials(part_o, part_lse):
    """Merge chunk partials by log-sum-exp weighting.

    part_o [rows, S, D] (each chunk's own normalised output), part_lse [rows, S]
    (each chunk's natural-log partition function, -inf for a chunk with no mass).
    m* = max_c lse_c, w_c = e^(lse_c - m*), out = sum w_c o_c / sum w_c,
    lse = m* + ln sum w_c.  A row whose chunks all have -inf gets out 0, lse -inf.
    """
    po = _f64(part_o); pl = _f64(part_lse)
    mstar = pl.max(axis=1)
    dead = np.isneginf(mstar)
    ms = np.where(dead, 0.0, mstar)
    w = np.exp(pl - ms[:, None])                             # -inf chunk -> weight 0
    wsum = w.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(dead[:, None], 0.0,
                       np.einsum("rs,rsd->rd", w, po) / np.where(dead, 1.0, wsum)[:, None])
        lse = np.where(dead, -np.inf, ms + np.log(np.where(dead, 1.0, wsum)))
    return out, lse


def sink_attention_chunked(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, sm_scale: float,
                           causal: bool, bounds: Sequence[Sequence[int]],
                           sink_chunks: str = "first", return_partials: bool = False):
    """Split-KV form: per-chunk partial softmax, then the log-sum-exp merge.

    bounds[b] = [a_0=0, a_1, ..., a_n=Lk_b], chunk c covers keys [a_c, a_{c+1}).
    Chunk c of a row has M_c = max([c==0]*sink, max s_j), Z_c = [c==0]*e^(sink-M_c) +
    sum e^(s_j-M_c), o_c = sum e^(s_j-M_c) v_j / Z_c, lse_c = M_c + ln Z_c.  The sink
    joins the first block only ("Sink attention"); ``sink_chunks`` exists so tests can
    show that the other choices ("all", "none") give a different, wrong answer.
    Every sequence must have the same number of chunks.
    Returns (out, lse) and, if return_partials, also (part_o [total_q, Hq, S, D],
    part_lse [total_q, Hq, S]).
    """
    q = _f64(q); k = _f64(k); v = _f64(v)
    cq = _i64(cu_seqlens_q); ck = _i64(cu_seqlens_kv)
    tq, hq, d = q.shape
    hkv = k.shape[0]
    gsz = hq // hkv
    nchunk = len(bounds[0]) - 1
    assert all(len(bd) - 1 == nchunk for bd in bounds)
    sig_all = np.full(hq, -np.inf) if sinks is None else _f64(sinks).reshape(hq)
    neg = np.full(hq, -np.inf)
    part_o = np.zeros((tq, hq, nchunk, d))
    part_l = np.full((tq, hq, nchunk), -np.inf)
    for b in range(len(cq) - 1):
        q0, q1 = int(cq[b]), int(cq[b + 1])
        k0, k1 = int(ck[b]), int(ck[b + 1])
        lq, lk = q1 - q0, k1 - k0
        bd = list(bounds[b])
        assert bd[0] == 0 and bd[-1] == lk
        for c in range(nchunk):
            a0, a1 = bd[c], bd[c + 1]
            use_sink = (sink_chunks == "all") or (sink_chunks == "first" and c == 0)
            sig_c = sig_all if use_sink else neg
            for g in range(hkv):
                heads = slice(g * gsz, (g + 1) * gsz)
                kb = k[g, k0 + a0:k0 + a1, :]
                vb = v[g, k0 + a0:k0 + a1, :]
                qb = np.transpose(q[q0:q1, heads, :], (1, 0, 2))
                s = (qb @ kb.T) * sm_scale
                vis = _visible(lq, lk, 0, lq, causal)[:, a0:a1]
                o, l = _softmax_with_sink(s, vis, sig_c[heads], vb)
                part_o[q0:q1, heads, c, :] = np.transpose(o, (1, 0, 2))
                part_l[q0:q1, heads, c] = l.T
    out, lse = merge_partials(part_o.reshape(tq * hq, nchunk, d),
                              part_l.reshape(tq * hq, nchunk))
    out = out.reshape(tq, hq, d)
    lse = lse.reshape(tq, hq)
    if return_partials:
        return out, lse, part_o, part_l
    return out, lse


def flops_causal(cu_seqlens_q, cu_seqlens_kv, num_q_heads: int, head_dim: int,
                 causal: bool = True) -> int:
    """Algorithmic flops of the two contractions: 4 * D * Hq * (visible query-key
    pairs).  Softmax and masked pairs are not counted."""
    cq = _i64(cu_seqlens_q); ck = _i64(cu_seqlens_kv)
    pairs = 0
    for b in range(len(cq) - 1):
        lq = int(cq[b + 1] - cq[b]); lk = int(ck[b + 1] - ck[b])
        if not causal:
            pairs += lq * lk
            continue
        for i in range(lq):
            pairs += max(0, min(lk, i + lk - lq + 1))
    return 4 * head_dim * num_q_heads * pairs
