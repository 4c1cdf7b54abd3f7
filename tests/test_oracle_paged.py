"""Pins of the paged-KV oracle (CPU): the page-table reading written out by hand, a
scatter built independently of the oracle's gather, append against concatenation,
and paged decode against the contiguous definition."""
import numpy as np
import pytest

from oracle import (gather_paged, kv_append, paged_seq_lens, sink_attention_decode,
                    sink_attention_decode_paged)


def _cache(num_pages, hkv, ps, d, fill):
    return np.full((num_pages, hkv, ps, d), fill, dtype=np.float64)


def test_hand_example_gather():
    # page_size 2, 1 KV head, head_dim 1.  Sequence 0: pages [3, 0], last page holds 1
    # token -> 3 tokens; sequence 1: pages [] -> empty; sequence 2: page [2], full.
    ps = 2
    cache = np.zeros((4, 1, ps, 1))
    cache[3, 0, :, 0] = [10, 11]
    cache[0, 0, :, 0] = [12, 99]      # slot 1 is past sequence 0's end
    cache[2, 0, :, 0] = [20, 21]
    cache[1, 0, :, 0] = [77, 78]      # owned by nobody
    indptr = [0, 2, 2, 3]
    indices = [3, 0, 2]
    last = [1, 2, 2]
    assert list(paged_seq_lens(indptr, last, ps)) == [3, 0, 2]
    out, kv_indptr = gather_paged(cache, indptr, indices, last, ps)
    assert list(kv_indptr) == [0, 3, 3, 5]
    assert out[0, :, 0].tolist() == [10, 11, 12, 20, 21]


def _scatter(contig, lens, ps, hkv, d, rng, spare=3):
    """Independent construction of a page table for contiguous HND tokens: pages are
    assigned from a random permutation, tokens are written slot by slot."""
    npages = [-(-lk // ps) for lk in lens]
    total = sum(npages) + spare
    perm = rng.permutation(total)
    cache = rng.standard_normal((total, hkv, ps, d))  # garbage everywhere first
    indptr, indices, last = [0], [], []
    base, p = 0, 0
    for lk, n in zip(lens, npages):
        pages = perm[p:p + n].tolist()
        p += n
        for t in range(lk):
            cache[pages[t // ps], :, t % ps, :] = contig[:, base + t, :]
        base += lk
        indices += pages
        indptr.append(len(indices))
        last.append(lk - (n - 1) * ps if n else 0)
    return cache, indptr, indices, last


def test_gather_inverts_independent_scatter():
    rng = np.random.default_rng(1)
    lens, hkv, d, ps = [5, 0, 16, 1, 33], 3, 4, 8
    contig = rng.standard_normal((hkv, sum(lens), d))
    cache, indptr, indices, last = _scatter(contig, lens, ps, hkv, d, rng)
    out, kv_indptr = gather_paged(cache, indptr, indices, last, ps)
    assert np.array_equal(out, contig)
    assert list(kv_indptr) == [0, 5, 5, 21, 22, 55]


def test_append_equals_concatenation():
    rng = np.random.default_rng(2)
    old, new, hkv, d, ps = [3, 0, 16, 7], [1, 4, 2, 9], 2, 4, 4
    full = [o + n for o, n in zip(old, new)]
    contig = rng.standard_normal((hkv, sum(full), d))
    cache_full, indptr, indices, last = _scatter(contig, full, ps, hkv, d, rng)
    # the cache before the append: the new positions hold garbage
    kc = cache_full.copy()
    base = 0
    newk = []
    for b, (o, n) in enumerate(zip(old, new)):
        for t in range(o, o + n):
            page = indices[indptr[b] + t // ps]
            kc[page, :, t % ps, :] = 1e9
        newk.append(contig[:, base + o: base + o + n, :].transpose(1, 0, 2))
        base += o + n
    k_new = np.concatenate(newk, axis=0)          # [total_new, Hkv, D]
    app = np.concatenate([[0], np.cumsum(new)])
    kc2, vc2 = kv_append(kc, kc, k_new, k_new, app, indptr, indices, last, ps)
    out, _ = gather_paged(kc2, indptr, indices, last, ps)
    assert np.array_equal(out, contig)
    assert np.array_equal(kc2, vc2)


@pytest.mark.parametrize("causal", [True, False])
def test_paged_decode_equals_contiguous(causal):
    rng = np.random.default_rng(3)
    lens, ql, hq, hkv, d, ps = [6, 1, 40, 17], 2, 8, 2, 16, 16
    lens = [max(lk, ql) for lk in lens]
    k = rng.standard_normal((hkv, sum(lens), d))
    v = rng.standard_normal((hkv, sum(lens), d))
    q = rng.standard_normal((len(lens), ql, hq, d))
    sinks = rng.standard_normal(hq)
    kc, indptr, indices, last = _scatter(k, lens, ps, hkv, d, np.random.default_rng(9))
    vc, indptr2, indices2, last2 = _scatter(v, lens, ps, hkv, d, np.random.default_rng(9))
    assert indices == indices2
    kv_indptr = np.concatenate([[0], np.cumsum(lens)])
    ro, rl = sink_attention_decode(q, k, v, sinks, kv_indptr, 0.25, causal)
    po, pl = sink_attention_decode_paged(q, kc, vc, sinks, indptr, indices, last, ps, 0.25,
                                         causal)
    assert np.array_equal(ro, po) and np.array_equal(rl, pl)
