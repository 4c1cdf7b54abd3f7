"""Seeded synthetic inputs for sink-aware GQA attention.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through the tests and the bench) and the
CPU oracle consume what it produces, and neither is imported here.

Recipe: one ``torch.Generator`` seeded with the workload's seed; draws in the fixed
order lengths -> Q -> K -> V -> sinks; Q/K/V are standard-normal float32 draws rounded
to bfloat16 (round to nearest even); sinks stay float32.  K and V are head-major
("HND", ``[kv_head, token, head_dim]``, tokens contiguous per head), the layout the
"Hosting Qwen on Blackwell" page gives its KV caches.  Prefill Q is token-major
``[total_q, Hq, D]``; decode Q is ``[batch, q_len, Hq, D]``.

The five named workloads follow the shapes of the pages' workloads: a tiny prefill,
gpt-oss-like decode (64 query heads over 8 KV heads, head_dim 64), a mixed-length
prefill, a ~6000-token prefill over 4 KV heads (head_dim 128), multi-token
(speculative) decode over 32768 cached tokens, and a chunked prefill (a 1024-token chunk
over a 31744-token cached prefix, the way long inputs are prefilled in pieces).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

__all__ = ["Workload", "CONFIGS", "make", "make_prefill", "make_decode", "seed_of"]

# name -> recipe.  Lengths are inclusive integer ranges; sink specs are
# ("normal", mean, std) or ("alt_neginf", mean, std): even query heads -inf, odd heads
# drawn from N(mean, std).
CONFIGS = {
    "tiny_prefill": dict(kind="prefill", batch=1, lens=(128, 128), hq=4, hkv=1, d=64,
                         sink=("normal", 0.0, 1.0), scale=1 / 8, causal=True),
    "decode_gptoss": dict(kind="decode", batch=64, q_len=1, hq=64, hkv=8, d=64,
                          lens=(1024, 8192), sink=("normal", 0.0, 2.0), scale=1 / 8,
                          causal=True, num_splits=0),
    "varlen_prefill": dict(kind="prefill", batch=8, lens=(512, 6000), hq=64, hkv=8, d=64,
                           sink=("normal", 0.0, 2.0), scale=1 / 8, causal=True),
    "long_prefill": dict(kind="prefill", batch=1, lens=(6000, 6000), hq=64, hkv=4, d=128,
                         sink=("alt_neginf", 2.0, 1.0), scale=1 / math.sqrt(128),
                         causal=True),
    "spec_decode": dict(kind="decode", batch=256, q_len=4, hq=64, hkv=4, d=128,
                        lens=(32768, 32768), sink=("normal", 0.0, 2.0),
                        scale=1 / math.sqrt(128), causal=True, num_splits=32),
    # chunked prefill: a 1024-token chunk over a 31744-token cached prefix
    "chunked_prefill": dict(kind="prefill", batch=1, lens=(1024, 1024), prefix=31744, hq=64,
                            hkv=8, d=64, sink=("normal", 0.0, 2.0), scale=1 / 8, causal=True),
}
_ORDER = list(CONFIGS)


def seed_of(name: str) -> int:
    """Seed of a named workload: 1234 + its 1-based position in CONFIGS."""
    return 1234 + 1 + _ORDER.index(name)


@dataclass
class Workload:
    kind: str                      # "prefill" or "decode"
    q: torch.Tensor                # bf16
    k: torch.Tensor                # bf16 [Hkv, total_kv, D]
    v: torch.Tensor                # bf16 [Hkv, total_kv, D]
    sinks: Optional[torch.Tensor]  # fp32 [Hq] or None
    cu_seqlens_q: torch.Tensor     # int32 [B+1] (decode: arange * q_len)
    cu_seqlens_kv: torch.Tensor    # int32 [B+1] (decode: kv_indptr)
    lens_q: list
    lens_kv: list
    hq: int
    hkv: int
    d: int
    scale: float
    causal: bool
    q_len: int = 0                 # decode only
    num_splits: int = 0            # decode only
    seed: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.lens_kv)

    @property
    def max_q(self) -> int:
        return max(self.lens_q) if self.lens_q else 0

    @property
    def max_kv(self) -> int:
        return max(self.lens_kv) if self.lens_kv else 0


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn_bf16(shape, gen, device, chunk=1 << 27) -> torch.Tensor:
    """N(0,1) float32 draws rounded to bf16, drawn in slices to bound scratch memory."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device,
                                dtype=torch.float32).to(torch.bfloat16)
    return out


def _sinks(spec, hq, gen, device) -> Optional[torch.Tensor]:
    if spec is None:
        return None
    kind, mean, std = spec
    z = torch.randn(hq, generator=gen, device=device, dtype=torch.float32) * std + mean
    if kind == "normal":
        return z
    if kind == "alt_neginf":
        z[0::2] = float("-inf")
        return z
    if kind == "neginf":
        return torch.full((hq,), float("-inf"), device=device)
    raise ValueError(kind)


def _lens(batch, lo_hi, gen):
    lo, hi = lo_hi
    if lo == hi:
        return [int(lo)] * batch
    return [int(x) for x in torch.randint(lo, hi + 1, (batch,), generator=gen)]


def _cumsum(lens, device):
    cu = [0]
    for x in lens:
        cu.append(cu[-1] + int(x))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def make_prefill(lens_q, lens_kv, hq, hkv, d, sink, scale, causal, seed, device="cpu",
                 name="") -> Workload:
    """Prefill workload with explicit per-sequence query and key lengths."""
    g = _gen(device, seed)
    tq, tk = sum(lens_q), sum(lens_kv)
    q = _randn_bf16((tq, hq, d), g, device)
    k = _randn_bf16((hkv, tk, d), g, device)
    v = _randn_bf16((hkv, tk, d), g, device)
    s = _sinks(sink, hq, g, device)
    return Workload("prefill", q, k, v, s, _cumsum(lens_q, device), _cumsum(lens_kv, device),
                    list(lens_q), list(lens_kv), hq, hkv, d, float(scale), bool(causal),
                    seed=seed, name=name)


def make_decode(lens_kv, q_len, hq, hkv, d, sink, scale, causal, num_splits, seed,
                device="cpu", name="") -> Workload:
    """Decode workload: q_len query tokens per sequence, KV lengths lens_kv (the KV
    already holds the q_len new tokens)."""
    g = _gen(device, seed)
    b = len(lens_kv)
    q = _randn_bf16((b, q_len, hq, d), g, device)
    tk = sum(lens_kv)
    k = _randn_bf16((hkv, tk, d), g, device)
    v = _randn_bf16((hkv, tk, d), g, device)
    s = _sinks(sink, hq, g, device)
    cu_q = torch.arange(b + 1, dtype=torch.int32, device=device) * q_len
    return Workload("decode", q, k, v, s, cu_q, _cumsum(lens_kv, device), [q_len] * b,
                    list(lens_kv), hq, hkv, d, float(scale), bool(causal), q_len=q_len,
                    num_splits=num_splits, seed=seed, name=name)


def make(name: str, device="cpu", seed: Optional[int] = None, **override) -> Workload:
    """Build a named workload.  ``override`` replaces recipe fields (e.g. a smaller
    batch for a test); lengths are drawn on the CPU generator before anything else so
    that they do not depend on the device."""
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    seed = seed_of(name) if seed is None else seed
    lens = _lens(cfg["batch"], cfg["lens"], _gen("cpu", seed))
    if cfg["kind"] == "prefill":
        lens_kv = [x + cfg.get("prefix", 0) for x in lens]
        w = make_prefill(lens, lens_kv, cfg["hq"], cfg["hkv"], cfg["d"], cfg["sink"],
                         cfg["scale"], cfg["causal"], seed + 7919, device, name)
    else:
        w = make_decode(lens, cfg["q_len"], cfg["hq"], cfg["hkv"], cfg["d"], cfg["sink"],
                        cfg["scale"], cfg["causal"], cfg["num_splits"], seed + 7919,
                        device, name)
    w.seed = seed
    return w


@dataclass
class PagedKV:
    """A paged copy of a workload's K/V: caches [num_pages, Hkv, page_size, D] (HND
    inside a page) and the page table that maps every sequence's tokens to pages."""
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    kv_page_indptr: torch.Tensor     # int32 [B+1]
    kv_page_indices: torch.Tensor    # int32 [entries]
    kv_last_page_len: torch.Tensor   # int32 [B]
    page_size: int

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]


def make_paged(w: "Workload", page_size: int, seed: int, spare_pages: int = 7,
               fill: str = "randn") -> PagedKV:
    """Scatter a workload's K/V into a paged cache.  Page ids come from a seeded
    permutation (so a sequence's pages are scattered over the cache) and ``spare_pages``
    pages belong to no sequence.  Slots no token occupies hold ``fill``: "randn" (bf16
    draws) or "nan"."""
    device = w.k.device
    gen = torch.Generator(device="cpu").manual_seed(seed)
    npages = [-(-lk // page_size) for lk in w.lens_kv]
    total = sum(npages) + spare_pages
    perm = torch.randperm(total, generator=gen)
    hkv, d = w.hkv, w.d
    if fill == "nan":
        kc = torch.full((total, hkv, page_size, d), float("nan"), dtype=torch.bfloat16,
                        device=device)
        vc = kc.clone()
    else:
        g2 = _gen(device, seed + 1)
        kc = _randn_bf16((total, hkv, page_size, d), g2, device)
        vc = _randn_bf16((total, hkv, page_size, d), g2, device)
    indptr, indices, last = [0], [], []
    tok_page, tok_slot = [], []
    p = 0
    for lk, n in zip(w.lens_kv, npages):
        pages = perm[p:p + n].tolist()
        p += n
        indices += pages
        indptr.append(len(indices))
        last.append(lk - (n - 1) * page_size if n else 0)
        for t in range(lk):
            tok_page.append(pages[t // page_size])
            tok_slot.append(t % page_size)
    if tok_page:
        tp = torch.tensor(tok_page, dtype=torch.long, device=device)
        ts = torch.tensor(tok_slot, dtype=torch.long, device=device)
        # [pages, ps, Hkv, D] views of the caches receive the token-major K/V rows
        kc.permute(0, 2, 1, 3)[tp, ts] = w.k.permute(1, 0, 2)
        vc.permute(0, 2, 1, 3)[tp, ts] = w.v.permute(1, 0, 2)
    as_i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=device)  # noqa: E731
    return PagedKV(kc, vc, as_i32(indptr), as_i32(indices if indices else [0]), as_i32(last),
                   page_size)
