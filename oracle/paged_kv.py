"""Paged HND KV cache: plain CPU reference of the page layout, of appending new tokens,
and of sink attention over a paged cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may call it.  It shares no code with the HIP kernels or their host runtime.

Layout (readings; the pages fix only part of it)
------------------------------------------------
"Hosting Qwen on Blackwell" (introduction) keeps KV caches head-major ("HND") so a cache
can be split or concatenated by head; "GPT-OSS on day 0" ("Kernels for GPT-OSS") adds the
sink to the attention templates of a paged-KV attention library.  Reading used here,
in that library's page-table convention:

* a cache is ``[num_pages, Hkv, page_size, D]``: inside a page, heads lead and each
  head's tokens are contiguous;
* sequence ``b`` owns the pages ``kv_page_indices[kv_page_indptr[b] :
  kv_page_indptr[b+1]]``, in order; with ``n_b`` pages its length is
  ``(n_b - 1) * page_size + kv_last_page_len[b]`` (0 when ``n_b == 0``);
* token ``t`` of sequence ``b`` lives in page ``kv_page_indices[kv_page_indptr[b] +
  t // page_size]`` at slot ``t % page_size``;
* appending ``n_b`` new tokens to sequence ``b`` writes them at positions
  ``L_b - n_b .. L_b - 1`` where ``L_b`` is the length the page table describes
  (the table already includes the new tokens).
"""
from __future__ import annotations

import numpy as np

from .sink_attention import _f64, _i64, sink_attention_decode

__all__ = ["paged_seq_lens", "gather_paged", "kv_append", "sink_attention_decode_paged"]


def paged_seq_lens(kv_page_indptr, kv_last_page_len, page_size: int) -> np.ndarray:
    """Length of every sequence described by a page table."""
    ind = _i64(kv_page_indptr)
    last = _i64(kv_last_page_len)
    n = ind[1:] - ind[:-1]
    return np.where(n > 0, (n - 1) * page_size + last, 0)


def gather_paged(cache, kv_page_indptr, kv_page_indices, kv_last_page_len, page_size: int):
    """Contiguous HND copy ``[Hkv, sum L_b, D]`` (float64) of the tokens a page table
    describes, sequences back to back, plus the matching ``kv_indptr`` ``[B+1]``."""
    c = _f64(cache)
    ind = _i64(kv_page_indptr)
    idx = _i64(kv_page_indices)
    lens = paged_seq_lens(ind, kv_last_page_len, page_size)
    hkv, d = c.shape[1], c.shape[3]
    out = np.zeros((hkv, int(lens.sum()), d))
    pos = 0
    for b in range(len(lens)):
        for t in range(int(lens[b])):
            page = idx[ind[b] + t // page_size]
            out[:, pos, :] = c[page, :, t % page_size, :]
            pos += 1
    kv_indptr = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return out, kv_indptr


def kv_append(k_cache, v_cache, k_new, v_new, append_indptr, kv_page_indptr,
              kv_page_indices, kv_last_page_len, page_size: int):
    """Caches (float64 copies) after writing the new tokens: ``k_new``/``v_new`` are
    ``[total_new, Hkv, D]`` (token-major, as a projection produces them) and sequence
    ``b`` owns rows ``append_indptr[b] : append_indptr[b+1]`` of them."""
    kc = _f64(k_cache).copy()
    vc = _f64(v_cache).copy()
    kn = _f64(k_new)
    vn = _f64(v_new)
    app = _i64(append_indptr)
    ind = _i64(kv_page_indptr)
    idx = _i64(kv_page_indices)
    lens = paged_seq_lens(ind, kv_last_page_len, page_size)
    for b in range(len(lens)):
        n_new = app[b + 1] - app[b]
        for i in range(int(n_new)):
            t = int(lens[b] - n_new + i)
            page = idx[ind[b] + t // page_size]
            kc[page, :, t % page_size, :] = kn[app[b] + i]
            vc[page, :, t % page_size, :] = vn[app[b] + i]
    return kc, vc


def sink_attention_decode_paged(q, k_cache, v_cache, sinks, kv_page_indptr, kv_page_indices,
                                kv_last_page_len, page_size: int, sm_scale: float,
                                causal: bool = True):
    """Decode attention over a paged cache: the sequences' tokens gathered in order,
    then the contiguous decode definition ("Sink attention")."""
    k, kv_indptr = gather_paged(k_cache, kv_page_indptr, kv_page_indices, kv_last_page_len,
                                page_size)
    v, _ = gather_paged(v_cache, kv_page_indptr, kv_page_indices, kv_last_page_len, page_size)
    return sink_attention_decode(q, k, v, sinks, kv_indptr, sm_scale, causal)
