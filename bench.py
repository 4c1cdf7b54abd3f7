"""Throughput of sink-aware GQA attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--only LINE]
                    [--no-cpu-baseline] [--no-others]

One step is one pass of the whole decode hot path (the split-KV kernel, every chunk
with its own online softmax and the sink in chunk 0, and the log-sum-exp merge) over
the large-batch speculative decode workload as it is named: 256 sequences x 4 draft
tokens (causal within the draft), 64 query heads over 4 KV heads, head_dim 128, 32768
cached keys each, 32 KV chunks per sequence.  Inputs are resident in HBM.  Before every
step a 512 MiB read (a sum over a scratch buffer) evicts the 256 MB Infinity Cache and
the L2s with clean lines, so each step streams its K/V from HBM; only the attention
call sits inside the timed event pair.  Times are the median (and minimum, and mean) of
the K timed steps.

The same JSON line carries the other workloads under "others" (the gpt-oss-like decode
batch, the speculative batch under the planner, varlen / long / chunked / tiny prefill
in TFLOP/s, decode over a paged cache and the paged KV append in GB/s), each with the
roofline of its dominant kernel and the fp64 CPU oracle timed on a bounded sample of
the same workload, and "peaks": the HBM rate of a flat read of the headline's K/V bytes
and the bf16 rate of a register-only MFMA loop, measured beside the spec-sheet peaks.

Algorithmic work (implementation overheads such as split partials are not counted):
  decode bytes  = K+V of every visible key once per KV head + Q + out + lse + sinks +
                  kv_indptr;  first-step kernel bytes = the same minus out and lse.
  prefill flops = 4 * head_dim * Hq * (visible query-key pairs).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FLUSH_BYTES = 512 << 20
CPU_BUDGET_HEADLINE_S = 10.0
CPU_BUDGET_LINE_S = 3.0


def _say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work
def _pairs(lens_q, lens_kv, causal):
    tot = 0
    for lq, lk in zip(lens_q, lens_kv):
        if not causal:
            tot += lq * lk
            continue
        i = np.arange(lq, dtype=np.int64)
        tot += int(np.clip(i + lk - lq + 1, 0, lk).sum())
    return tot


def decode_bytes(w, first_step_only=False):
    kv = sum(w.lens_kv) * w.hkv * w.d * 2 * 2
    q = w.q.numel() * 2
    small = w.hq * 4 + (w.batch + 1) * 4
    if first_step_only:
        return kv + q + small
    return kv + q + q + w.batch * w.q_len * w.hq * 4 + small


def prefill_flops(w):
    return 4 * w.d * w.hq * _pairs(w.lens_q, w.lens_kv, w.causal)


# ---------------------------------------------------------------- timing
class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, n, marks=2):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(marks)] for _ in range(n)]

    def mark(self, i, j):
        self.ev[i][j].record(torch.cuda.current_stream())

    def ms(self, j0, j1):
        return [e[j0].elapsed_time(e[j1]) for e in self.ev]


def stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return dict(median=float(np.median(a)), min=float(a.min()), mean=float(a.mean()), n=len(a))


def time_calls(fns, steps, warmup, flush):
    """Event times of one step = the calls in `fns` back to back (a cache flush before
    each step; an event before the first call and after each one).  Returns one stats
    dict for the whole step and one per call."""
    for _ in range(warmup):
        flush.sum()
        for f in fns:
            f()
    torch.cuda.synchronize()
    t = Timer(steps, len(fns) + 1)
    for i in range(steps):
        flush.sum()
        t.mark(i, 0)
        for j, f in enumerate(fns):
            f()
            t.mark(i, j + 1)
    torch.cuda.synchronize()
    return stats(t.ms(0, len(fns))), [stats(t.ms(j, j + 1)) for j in range(len(fns))]


def _c_call(fn, args):
    """A pre-marshalled C-ABI call: no Python argument handling between the events."""
    def call():
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{fn.__name__} failed with status {rc}")
    return call


def _source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gqa_attention_sink_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _traffic_for(kernel, workload):
    """HBM bytes per launch that rocprofv3 counters measured for this kernel and
    workload (profiles/traffic.json), if taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{kernel}:{workload}")
    except Exception:
        return None
    if not rec or rec.get("source_hash") != _source_hash():
        return None
    return rec.get("bytes_per_launch")


def _r(x, n=4):
    return None if x is None else round(float(x), n)


# ---------------------------------------------------------------- host facts
def host_info():
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = len(os.sched_getaffinity(0))
    return dict(cpu_model=model, host_cpus=len(os.sched_getaffinity(0)), blas_threads=int(blas))


HOST = None


def _baseline(value, unit, t_used, sample):
    return {"value": round(value, 6), "unit": unit, "cores": HOST["blas_threads"],
            "kind": "oracle", "cpu_model": HOST["cpu_model"], "host_cpus": HOST["host_cpus"],
            "sample": f"{sample}; {t_used:.1f} s of fp64 numpy on the host"}


# ---------------------------------------------------------------- CPU oracle samples
def cpu_decode(w, budget_s):
    """The oracle on whole sequences of a decode workload (all heads), in order, until
    about budget_s seconds of CPU work; GB/s of the sample's algorithmic bytes."""
    import oracle
    ind = w.cu_seqlens_kv.cpu().tolist()
    done, t_used, n = 0, 0.0, 0
    for b in range(w.batch):
        lk = ind[b + 1] - ind[b]
        q = w.q[b:b + 1].cpu()
        k = w.k[:, ind[b]:ind[b + 1]].cpu()
        v = w.v[:, ind[b]:ind[b + 1]].cpu()
        t0 = time.perf_counter()
        oracle.sink_attention_decode(q, k, v, w.sinks, [0, lk], w.scale, w.causal)
        t_used += time.perf_counter() - t0
        done += lk * w.hkv * w.d * 4 + 2 * q.numel() * 2 + w.q_len * w.hq * 4
        n += 1
        if t_used >= budget_s:
            break
    return _baseline(done / t_used / 1e9, "GB/s", t_used,
                     f"{n} of {w.batch} sequences of {w.name} (all heads)")


def cpu_prefill(w, budget_s, rows=128):
    """The oracle on blocks of `rows` query rows (all heads) with the keys they see,
    the last block of each sequence first, until about budget_s seconds; TFLOP/s of the
    sample's causal pairs."""
    import oracle
    cq = w.cu_seqlens_q.cpu().tolist()
    ck = w.cu_seqlens_kv.cpu().tolist()
    blocks = []
    for b in range(w.batch):
        lq = cq[b + 1] - cq[b]
        for r1 in range(lq, 0, -rows):
            blocks.append((b, max(0, r1 - rows), r1))
    # interleave sequences so the sample spans them
    blocks.sort(key=lambda x: (x[2] - x[1] < rows, -(x[2]), x[0]))
    flops, t_used, n = 0, 0.0, 0
    for b, r0, r1 in blocks:
        lq, lk = cq[b + 1] - cq[b], ck[b + 1] - ck[b]
        off = lk - lq
        nk = min(lk, r1 + off) if w.causal else lk
        q = w.q[cq[b] + r0:cq[b] + r1].cpu()
        k = w.k[:, ck[b]:ck[b] + nk].cpu()
        v = w.v[:, ck[b]:ck[b] + nk].cpu()
        t0 = time.perf_counter()
        oracle.sink_attention(q, k, v, w.sinks, [0, r1 - r0], [0, nk], w.scale, w.causal)
        t_used += time.perf_counter() - t0
        flops += 4 * w.d * w.hq * _pairs([r1 - r0], [nk], w.causal)
        n += 1
        if t_used >= budget_s:
            break
    return _baseline(flops / t_used / 1e12, "TFLOP/s", t_used,
                     f"{n} blocks of <= {rows} query rows of {w.name} (all heads)")


def cpu_paged(w, pk, page_size, budget_s, rope=None):
    """The paged-cache oracle on whole sequences: their pages copied into a small host
    cache with their own page table (with `rope`, the oracle's YaRN rotation of the
    queries at positions Lk - q_len + t first); GB/s of the sample's algorithmic bytes."""
    import oracle
    ind = pk.kv_page_indptr.cpu().tolist()
    idx = pk.kv_page_indices.cpu().tolist()
    last = pk.kv_last_page_len.cpu().tolist()
    done, t_used, n = 0, 0.0, 0
    for b in range(w.batch):
        pages = idx[ind[b]:ind[b + 1]]
        kc = pk.k_cache[pages].cpu()
        vc = pk.v_cache[pages].cpu()
        q = w.q[b:b + 1].cpu()
        lk = (len(pages) - 1) * page_size + last[b] if pages else 0
        t0 = time.perf_counter()
        if rope is not None:
            pos = (lk - w.q_len + np.arange(w.q_len))[None, :, None]
            q = oracle.bf16_round(oracle.apply_rope(q, pos, **rope))
        oracle.sink_attention_decode_paged(q, kc, vc, w.sinks, [0, len(pages)],
                                           list(range(len(pages))), [last[b]], page_size,
                                           w.scale, w.causal)
        t_used += time.perf_counter() - t0
        done += lk * w.hkv * w.d * 4 + 2 * w.q_len * w.hq * w.d * 2 + w.q_len * w.hq * 4 + len(pages) * 4
        n += 1
        if t_used >= budget_s:
            break
    return _baseline(done / t_used / 1e9, "GB/s", t_used,
                     f"{n} of {w.batch} sequences of {w.name} in {page_size}-token pages" +
                     (", queries rotated" if rope is not None else ""))


def cpu_append(p, pk, k_new, v_new, page_size, budget_s, rope=None):
    """The append oracle on whole sequences (their pages in a small host cache; with
    `rope`, the oracle's YaRN rotation of the new keys at their positions first); GB/s of
    the new K/V read and written."""
    import oracle
    ind = pk.kv_page_indptr.cpu().tolist()
    idx = pk.kv_page_indices.cpu().tolist()
    last = pk.kv_last_page_len.cpu().tolist()
    app = p.cu_seqlens_kv.cpu().tolist()
    done, t_used, n = 0, 0.0, 0
    for b in range(p.batch):
        pages = idx[ind[b]:ind[b + 1]]
        kc = pk.k_cache[pages].cpu()
        vc = pk.v_cache[pages].cpu()
        kn = k_new[app[b]:app[b + 1]].cpu()
        vn = v_new[app[b]:app[b + 1]].cpu()
        t0 = time.perf_counter()
        if rope is not None:
            lk = (len(pages) - 1) * page_size + last[b] if pages else 0
            pos = lk - kn.shape[0] + np.arange(kn.shape[0])
            kn = oracle.bf16_round(oracle.apply_rope(kn, pos[:, None], **rope))
        oracle.kv_append(kc, vc, kn, vn, [0, kn.shape[0]], [0, len(pages)],
                         list(range(len(pages))), [last[b]], page_size)
        t_used += time.perf_counter() - t0
        done += 2 * 2 * vn.numel() * 2
        n += 1
        if t_used >= budget_s:
            break
    return _baseline(done / t_used / 1e9, "GB/s", t_used,
                     f"{n} of {p.batch} sequences of the varlen K/V appended" +
                     (", keys rotated" if rope is not None else ""))


# ---------------------------------------------------------------- GPU lines
def decode_line(sa, w, steps, warmup, flush, cpu_budget):
    """Whole decode call, and its kernels alone (the same launches decode makes): the
    first (dominant) kernel gives the roofline; a one-slot plan is a single kernel."""
    from gqa_attention_sink_amd import sink_attn as sam
    lib = sam.load()
    P = sam._ptr
    st = sam._stream(w.q.device)
    ns = int(w.num_splits)
    ws = sa.decode_workspace(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, ns)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.q_len, w.hq), dtype=torch.float32, device="cuda")
    tk = w.k.shape[1]
    scale, causal, mk = float(w.scale), int(bool(w.causal)), int(w.max_kv)
    rows_per_head = w.q_len * (w.hq // w.hkv)
    kind = sa.decode_plan_kind(w.batch, w.q_len, w.hq, w.hkv, w.d, tk, mk, ns)
    plan = sa.decode_stream_plan(w.batch, w.q_len, w.hq, w.hkv, w.d, tk, mk) if kind == "stream" else None
    full = _c_call(lib.sink_attn_decode,
                   (P(w.q), P(w.k), P(w.v), P(w.sinks), P(w.cu_seqlens_kv), w.batch, w.q_len, tk,
                    mk, w.hq, w.hkv, w.d, scale, causal, ns, P(ws), ws.numel(), P(out), P(lse),
                    None, st))
    steps_alone = None
    if plan is not None:
        kname = "decode_stream_wg_kernel" if rows_per_head > 16 else "decode_stream_kernel"
        part = _c_call(lib.sink_attn_decode_stream_partial,
                       (P(w.q), P(w.k), P(w.v), P(w.cu_seqlens_kv), w.batch, w.q_len, tk, mk,
                        w.hq, w.hkv, w.d, scale, causal, P(ws), ws.numel(), None, st))
        merge = _c_call(lib.sink_attn_decode_stream_merge,
                        (P(w.sinks), P(w.cu_seqlens_kv), w.batch, w.q_len, tk, mk, w.hq, w.hkv,
                         w.d, P(ws), ws.numel(), P(out), P(lse), st))
        steps_alone = [part, merge]
        plan_desc = dict(kind="stream", range_tokens=plan[0], ranges_per_head=plan[1],
                         slots=plan[2])
    elif kind == "whole_runs":  # one slot: the split kernel writes the result
        slots = 1
        kname = "decode_split_kernel"
        plan_desc = dict(kind="whole_runs", chunks_per_slot="all", slots=1)
    else:
        slots = sa.decode_num_slots(w.batch, w.q_len, w.hq, w.hkv, w.d, mk, ns)
        cps = sa.decode_chunks_per_slot(w.batch, w.q_len, w.hq, w.hkv, w.d, mk, ns)
        kname = "decode_cw_kernel" if rows_per_head <= 16 else "decode_split_kernel"
        plan_desc = dict(kind="chunks", chunks_per_slot=cps, slots=slots)
        if slots > 1:
            rows = w.batch * w.q_len * w.hq
            po = torch.empty((rows, slots, w.d), dtype=torch.float32, device="cuda")
            pl = torch.empty((rows, slots), dtype=torch.float32, device="cuda")
            part = _c_call(lib.sink_attn_decode_partial,
                           (P(w.q), P(w.k), P(w.v), P(w.sinks), P(w.cu_seqlens_kv), w.batch,
                            w.q_len, tk, mk, w.hq, w.hkv, w.d, scale, causal, ns, P(po), P(pl),
                            None, st))
            merge = _c_call(lib.sink_attn_merge, (P(po), P(pl), None, rows, slots, w.d, P(out), P(lse), st))
            steps_alone = [part, merge]
    t0 = time.perf_counter()
    whole, _ = time_calls([full], steps, warmup, flush)
    wall = time.perf_counter() - t0
    nbytes = decode_bytes(w)
    gbs = nbytes / (whole["median"] * 1e-3) / 1e9
    if steps_alone is not None:
        _, (s_part, s_merge) = time_calls(steps_alone, steps, warmup, flush)
        kbytes = decode_bytes(w, True)
        k_ms, k_min, m_ms = s_part["median"], s_part["min"], s_merge["median"]
        note = "the first kernel alone (partials), then the merge"
    else:   # one slot: the kernel writes the result, so it is the whole call
        kbytes, k_ms, k_min, m_ms = nbytes, whole["median"], whole["min"], 0.0
        note = "one kernel writes the result (every chunk merged inside its workgroup)"
    kgbs = kbytes / (k_ms * 1e-3) / 1e9
    line = {"GB/s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "ms": _r(whole["median"]), "ms_min": _r(whole["min"]), "ms_mean": _r(whole["mean"]),
            "steps": whole["n"], "wall_s": round(wall, 3), "bytes": nbytes,
            "num_splits": ns,
            "plan": (f"{ns} chunks per sequence, each its own online softmax (sink in chunk "
                     "0), merged by log-sum-exp") if ns else
                    ("planner: every chunk of a sequence in one workgroup (equal lengths, "
                     "at least two workgroups per CU), merged inside it" if kind == "whole_runs"
                     else "planner: ranges of each KV head's token axis, sink added in the merge"),
            "slot_plan": plan_desc,
            "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(kgbs, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                         "traffic": _traffic_for(kname, w.name + (f"/{ns}" if ns else "")),
                         "algorithmic_bytes_per_launch": kbytes,
                         "avg_launch_ms": _r(k_ms), "launch_ms_min": _r(k_min),
                         "merge_ms": _r(m_ms), "note": note}}
    if cpu_budget:
        line["cpu_baseline"] = cpu_decode(w, cpu_budget)
    return line


def prefill_line(sa, w, steps, warmup, flush, cpu_budget, num_splits=1):
    from gqa_attention_sink_amd import sink_attn as sam
    lib = sam.load()
    P = sam._ptr
    st = sam._stream(w.q.device)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.q.shape[0], w.hq), dtype=torch.float32, device="cuda")
    tq, tk = w.q.shape[0], w.k.shape[1]
    common = (P(w.q), P(w.k), P(w.v), P(w.sinks), P(w.cu_seqlens_q), P(w.cu_seqlens_kv),
              w.batch, int(w.max_q))
    tail = (tq, tk, w.hq, w.hkv, w.d, float(w.scale), int(bool(w.causal)))
    ns = 1
    if num_splits == 1:
        call = _c_call(lib.sink_attn_prefill, common + tail + (P(out), P(lse), None, st))
    else:
        ns = sa.prefill_num_splits(w.batch, w.max_q, w.max_kv, w.hq, w.hkv, num_splits)
        ws = torch.empty(max(256, sa.prefill_workspace_bytes(tq, w.hq, w.d, ns)),
                         dtype=torch.uint8, device="cuda")
        call = _c_call(lib.sink_attn_prefill_split,
                       common + (int(w.max_kv),) + tail + (int(num_splits), P(ws), ws.numel(),
                                                           P(out), P(lse), None, st))
    whole, _ = time_calls([call], steps, warmup, flush)
    fl = prefill_flops(w)
    tf = fl / (whole["median"] * 1e-3) / 1e12
    kname = "prefill_kernel" if w.d == 64 else "prefill_pp_kernel"
    # HBM bytes if every tensor moved once: Q, K, V read, O and lse written
    min_bytes = 2 * tq * w.hq * w.d * 2 + 2 * tk * w.hkv * w.d * 2 + tq * w.hq * 4
    traffic = _traffic_for(kname, w.name)   # the prefill kernel's launch (not the merge)
    line = {"TFLOP/s": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "ms": _r(whole["median"]), "ms_min": _r(whole["min"]), "ms_mean": _r(whole["mean"]),
            "steps": whole["n"], "flops": fl, "key_splits": ns, "min_hbm_bytes": min_bytes,
            "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(tf, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                         "note": "whole call (one kernel" + (", plus the merge)" if ns > 1 else ")")}}
    if traffic:
        line["traffic_over_min_hbm_bytes"] = round(traffic / min_bytes, 3)
    if cpu_budget:
        line["cpu_baseline"] = cpu_prefill(w, cpu_budget)
    return line


# YaRN parameters of the rotated lines (32x over a 4096-token original context)
YARN_BENCH = dict(theta=150000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0,
                  beta_slow=1.0)


def paged_lines(sa, steps, warmup, flush, cpu_budget):
    """Decode over a paged cache (the gpt-oss-like batch, 16-token pages scattered by a
    seeded permutation) and the KV append of the varlen batch's K/V into a paged cache.
    Bytes are algorithmic: decode as the contiguous decode plus the page list; append =
    new K and V read once and written once."""
    from gqa_attention_sink_amd import sink_attn as sam
    from gqa_attention_sink_amd import workloads as wl
    lib = sam.load()
    P = sam._ptr
    st = sam._stream(torch.device("cuda"))

    def paged_call(w, pk, ws, out, lse, rope):
        """sink_attn_decode_paged with its arguments marshalled once (checked by one
        call through the binding first)."""
        sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,
                        pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale, w.causal,
                        w.num_splits, workspace=ws, out=out, lse=lse, rope=rope)
        npg, hkv, ps, d = pk.k_cache.shape[0], pk.k_cache.shape[1], pk.k_cache.shape[2], w.d
        return _c_call(lib.sink_attn_decode_paged,
                       (P(w.q), P(pk.k_cache), P(pk.v_cache), P(w.sinks), P(pk.kv_page_indptr),
                        P(pk.kv_page_indices), P(pk.kv_last_page_len), w.batch, w.q_len,
                        pk.kv_page_indices.numel(), npg, ps, int(w.max_kv), w.hq, hkv, d,
                        float(w.scale), int(bool(w.causal)), int(w.num_splits), P(ws), ws.numel(),
                        P(out), P(lse), None if rope is None else ctypes.byref(rope), st))

    res = {}
    w = wl.make("decode_gptoss", device="cuda")
    pk = wl.make_paged(w, 16, seed=4242)
    ws = sa.decode_workspace(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, w.num_splits)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.q_len, w.hq), dtype=torch.float32, device="cuda")
    nbytes = decode_bytes(w) + pk.kv_page_indices.numel() * 4 + w.batch * 4
    for name, rope in (("paged_decode", None), ("paged_decode_rope", sa.RopeParams(**YARN_BENCH))):
        fn = paged_call(w, pk, ws, out, lse, rope)
        s, _ = time_calls([fn], steps, warmup, flush)
        g = nbytes / (s["median"] * 1e-3) / 1e9
        res[name] = {"GB/s": round(g, 2), "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4),
                     "ms": _r(s["median"]), "ms_min": _r(s["min"]), "ms_mean": _r(s["mean"]),
                     "steps": s["n"], "page_size": 16, "bytes": nbytes,
                     "workload": "decode_gptoss in a paged cache" +
                                 (" with fused YaRN rotation of q" if rope else ""),
                     "roofline": {"bound": "hbm", "kernel": "decode_stream_kernel (paged)",
                                  "achieved": round(g, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(g / HBM_PEAK_GBS, 4),
                                  "traffic": None if rope else _traffic_for(
                                      "decode_stream_kernel_paged", "decode_gptoss_paged16"),
                                  "note": "whole call (stream kernel + merge); traffic: the "
                                          "stream kernel's launch"}}
        if rope:
            res[name]["rope"] = YARN_BENCH
    if cpu_budget:
        res["paged_decode"]["cpu_baseline"] = cpu_paged(w, pk, 16, cpu_budget)
        res["paged_decode_rope"]["cpu_baseline"] = cpu_paged(w, pk, 16, cpu_budget, YARN_BENCH)
    del pk, ws
    torch.cuda.empty_cache()
    # the speculative-decode batch in 16-token pages, planner mode
    w5 = wl.make("spec_decode", device="cuda")
    w5.num_splits = 0
    pk5 = wl.make_paged(w5, 16, seed=4242)
    w5.k = w5.v = None  # only the paged copy is read
    torch.cuda.empty_cache()
    kind = sa.decode_plan_kind(w5.batch, w5.q_len, w5.hq, w5.hkv, w5.d,
                               (pk5.kv_page_indices.numel() - w5.batch) * 16, w5.max_kv, 0)
    ws5 = sa.decode_workspace(w5.batch, w5.q_len, w5.hq, w5.hkv, w5.d, w5.max_kv, 0)
    out5 = torch.empty_like(w5.q)
    lse5 = torch.empty((w5.batch, w5.q_len, w5.hq), dtype=torch.float32, device="cuda")
    s, _ = time_calls([paged_call(w5, pk5, ws5, out5, lse5, None)], steps, warmup, flush)
    nb5 = decode_bytes(w5) + pk5.kv_page_indices.numel() * 4 + w5.batch * 4
    g = nb5 / (s["median"] * 1e-3) / 1e9
    kname = "decode_split_kernel" if kind == "whole_runs" else "decode_stream_wg_kernel"
    res["paged_spec_decode"] = {
        "GB/s": round(g, 2), "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4),
        "ms": _r(s["median"]), "ms_min": _r(s["min"]), "ms_mean": _r(s["mean"]),
        "steps": s["n"], "page_size": 16, "bytes": nb5, "plan": kind,
        "workload": "spec_decode in a paged cache, planner mode (num_splits = 0)",
        "roofline": {"bound": "hbm", "kernel": kname + " (paged)", "achieved": round(g, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(g / HBM_PEAK_GBS, 4),
                     "traffic": _traffic_for(kname + "_paged", "spec_decode_paged16"),
                     "note": "whole call (one kernel: every chunk of a sequence in one "
                             "workgroup, the result written directly)"
                             if kind == "whole_runs" else "whole call"}}
    if cpu_budget:
        res["paged_spec_decode"]["cpu_baseline"] = cpu_paged(w5, pk5, 16, cpu_budget)
    del w5, pk5, ws5, out5, lse5
    torch.cuda.empty_cache()
    p = wl.make("varlen_prefill", device="cuda")
    pk = wl.make_paged(p, 16, seed=4343)
    k_new = p.k.permute(1, 0, 2).contiguous()
    v_new = p.v.permute(1, 0, 2).contiguous()
    app = p.cu_seqlens_kv
    nbytes = 2 * 2 * k_new.numel() * 2
    for name, rope in (("kv_append", None), ("kv_append_rope", sa.RopeParams(**YARN_BENCH))):
        sa.kv_append(k_new, v_new, app, pk.kv_page_indptr, pk.kv_page_indices,
                     pk.kv_last_page_len, pk.k_cache, pk.v_cache, p.max_kv, rope=rope)
        fn = _c_call(lib.sink_attn_kv_append,
                     (P(k_new), P(v_new), P(app), P(pk.kv_page_indptr), P(pk.kv_page_indices),
                      P(pk.kv_last_page_len), p.batch, int(p.max_kv), k_new.shape[0],
                      pk.kv_page_indices.numel(), pk.k_cache.shape[0], 16, p.hkv, p.d,
                      P(pk.k_cache), P(pk.v_cache), None if rope is None else ctypes.byref(rope),
                      st))
        s, _ = time_calls([fn], steps, warmup, flush)
        g = nbytes / (s["median"] * 1e-3) / 1e9
        res[name] = {"GB/s": round(g, 2), "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4),
                     "ms": _r(s["median"]), "ms_min": _r(s["min"]), "ms_mean": _r(s["mean"]),
                     "steps": s["n"], "page_size": 16, "tokens": int(k_new.shape[0]),
                     "bytes": nbytes,
                     "workload": "varlen_prefill K/V appended to a paged cache" +
                                 (" with fused YaRN rotation of the keys" if rope else ""),
                     "roofline": {"bound": "hbm", "kernel": "kv_append_kernel",
                                  "achieved": round(g, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(g / HBM_PEAK_GBS, 4),
                                  "traffic": None if rope else _traffic_for("kv_append_kernel",
                                                                            "kv_append")}}
    if cpu_budget:
        res["kv_append"]["cpu_baseline"] = cpu_append(p, pk, k_new, v_new, 16, cpu_budget)
        res["kv_append_rope"]["cpu_baseline"] = cpu_append(p, pk, k_new, v_new, 16, cpu_budget,
                                                           YARN_BENCH)
    return res


def tiny_line(sa, steps, warmup, flush, cpu_budget):
    """The tiny prefill (128 tokens): launch-bound, reported as latency."""
    from gqa_attention_sink_amd import workloads as wl
    w = wl.make("tiny_prefill", device="cuda")
    line = prefill_line(sa, w, steps, warmup, flush, 0)
    line["latency_us"] = round(line["ms"] * 1e3, 2)
    if cpu_budget:
        import oracle
        t0 = time.perf_counter()
        oracle.sink_attention(w.q, w.k, w.v, w.sinks, w.cu_seqlens_q.cpu(), w.cu_seqlens_kv.cpu(),
                              w.scale, w.causal)
        t = time.perf_counter() - t0
        line["cpu_baseline"] = _baseline(prefill_flops(w) / t / 1e12, "TFLOP/s", t,
                                         "the whole workload")
        line["cpu_baseline"]["latency_us"] = round(t * 1e6, 1)
    return line


def peaks(w, steps, warmup, flush):
    """Achievable rates measured on this GPU: a flat non-temporal read of the headline's
    K and V (the same bytes, one launch each, every workgroup streaming one contiguous
    share), a register-only bf16 MFMA loop with two wavefronts per SIMD, the MFMA rate
    of one chain per SIMD beside 0-4 exp2+FMA pairs per MFMA (the softmax's vector work)
    issued by the same wavefront or by the other wavefront of the SIMD, and the issue rate
    of v_exp_f32 and v_fma_f32 with 1, 2 or 4 wavefronts per SIMD."""
    from gqa_attention_sink_amd import build as bld
    lib = ctypes.CDLL(bld.PEAK_LIB)
    lib.sink_attn_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                               ctypes.c_void_p, ctypes.c_void_p]
    lib.sink_attn_peak_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                             ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.zeros(4, dtype=torch.uint8, device="cuda")
    kb = w.k.numel() * 2
    rd = [_c_call(lib.sink_attn_peak_stream_read,
                  (ctypes.c_void_p(t.data_ptr()), kb, 4 * cus, ctypes.c_void_p(sink.data_ptr()), st))
          for t in (w.k, w.v)]
    s, _ = time_calls(rd, steps, warmup, flush)
    hbm = 2 * kb / (s["median"] * 1e-3) / 1e9
    iters, blocks = 2048, 2 * cus
    outb = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    mf = _c_call(lib.sink_attn_peak_mfma_bf16, (iters, blocks, ctypes.c_void_p(outb.data_ptr()), st))
    sm, _ = time_calls([mf], steps, warmup, flush)
    flops = blocks * 4 * iters * 8 * 32768
    tf = flops / (sm["median"] * 1e-3) / 1e12
    # one MFMA chain per SIMD with E exp2+FMA pairs per MFMA, issued by the same
    # wavefront or by a second wavefront on the SIMD
    lib.sink_attn_peak_coissue.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    cb, ci = cus, 1024
    outc = torch.empty(cb * 512, dtype=torch.float32, device="cuda")
    co = {"same_wavefront": {}, "other_wavefront": {}}
    for split, key in ((0, "same_wavefront"), (1, "other_wavefront")):
        for e in range(5):
            fn = _c_call(lib.sink_attn_peak_coissue, (e, split, ci, cb, ctypes.c_void_p(outc.data_ptr()), st))
            sc, _ = time_calls([fn], steps, warmup, flush)
            co[key][str(e)] = round(cb * 4 * ci * 8 * 32768 / (sc["median"] * 1e-3) / 1e12, 1)
    # vector issue rate of the softmax's two main instructions, 1, 2 or 4 wavefronts per SIMD
    lib.sink_attn_peak_valu.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    vi = 8192
    outv = torch.empty(cus * 1024, dtype=torch.float32, device="cuda")  # a float per lane, up to 1024 lanes a workgroup
    valu = {}
    for op, oname in ((0, "v_exp_f32"), (1, "v_fma_f32")):
        for wps in (1, 2, 4):
            fn = _c_call(lib.sink_attn_peak_valu, (op, wps, vi, cus, ctypes.c_void_p(outv.data_ptr()), st))
            time_calls([fn], steps, warmup, flush)
            torch.cuda.synchronize()
            # lane 0 of every wavefront: shader-clock cycles of its loop; wps wavefronts share
            # a SIMD, so the SIMD issued wps * vi * 8 instructions in that time
            cyc = outv[: cus * 256 * wps].view(cus, 4 * wps, 64)[:, :, 0].double()
            valu.setdefault(oname, {})[str(wps)] = round(float(cyc.median()) / (wps * vi * 8), 2)
    return {"hbm_flat_read": {"GB/s": round(hbm, 1), "frac_of_spec": round(hbm / HBM_PEAK_GBS, 4),
                              "bytes": 2 * kb, "ms": _r(s["median"]),
                              "what": f"non-temporal 16-byte loads over {w.name}'s K and V, "
                                      f"{4 * cus} workgroups each streaming a contiguous share"},
            "bf16_mfma_loop": {"TFLOP/s": round(tf, 1), "frac_of_spec": round(tf / BF16_PEAK_TFLOPS, 4),
                               "ms": _r(sm["median"]),
                               "what": f"{blocks} workgroups x 4 wavefronts, 8 independent "
                                       "32x32x16 MFMA chains each, no memory traffic"},
            "mfma_beside_exp_TFLOP/s": dict(co, what=f"{cb} workgroups, one 32x32x16 MFMA chain "
                                                     "per SIMD; key = exp2+FMA pairs per MFMA, "
                                                     "issued after each MFMA by the same "
                                                     "wavefront or by the SIMD's second one"),
            "valu_cycles_per_wave64_instr": dict(valu, what=f"{cus} workgroups, key = wavefronts "
                                                            "per SIMD, each issuing 8 independent "
                                                            "chains; shader-clock cycles per "
                                                            "instruction issued by the SIMD"),
            "compute_units": cus}


# ---------------------------------------------------------------- main
def main():
    global HOST
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="spec_decode", choices=["spec_decode", "decode_gptoss"])
    ap.add_argument("--only", default=None,
                    help="run one line only (for profiling): spec_decode, spec_decode_planner, "
                         "decode_gptoss, varlen_prefill, long_prefill, chunked_prefill, "
                         "tiny_prefill, paged, peaks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the reference "
                         "kernel for scaling HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(decode shards by sequence and prefill by head with no exchange inside "
              "attention); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return

    import gqa_attention_sink_amd as sa
    from gqa_attention_sink_amd import workloads as wl
    if not os.path.exists(sa.LIB_PATH):
        from gqa_attention_sink_amd.build import build
        build()
    sa.load()
    torch.cuda.set_device(0)
    HOST = host_info()
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    cpu_head = 0 if args.no_cpu_baseline else CPU_BUDGET_HEADLINE_S
    cpu_line = 0 if args.no_cpu_baseline else CPU_BUDGET_LINE_S
    S, W = args.steps, args.warmup

    if args.only:
        o = args.only
        if o in ("spec_decode", "decode_gptoss"):
            res = decode_line(sa, wl.make(o, device="cuda"), S, W, flush, cpu_line)
        elif o == "spec_decode_planner":
            w = wl.make("spec_decode", device="cuda")
            w.num_splits = 0
            res = decode_line(sa, w, S, W, flush, cpu_line)
        elif o in ("varlen_prefill", "long_prefill"):
            res = prefill_line(sa, wl.make(o, device="cuda"), S, W, flush, cpu_line)
        elif o == "chunked_prefill":
            res = prefill_line(sa, wl.make(o, device="cuda"), S, W, flush, cpu_line, num_splits=0)
        elif o == "tiny_prefill":
            res = tiny_line(sa, S, W, flush, cpu_line)
        elif o == "paged":
            res = paged_lines(sa, S, W, flush, cpu_line)
        elif o == "peaks":
            res = peaks(wl.make("spec_decode", device="cuda"), S, W, flush)
        else:
            raise SystemExit(f"unknown line {o}")
        print(json.dumps({"only": o, "result": res}), flush=True)
        return

    _say(f"workload {args.workload} (headline)")
    w = wl.make(args.workload, device="cuda")
    head = decode_line(sa, w, S, W, flush, cpu_head)
    line = {
        "metric": "sink-attn decode HBM GB/s (and prefill TFLOP/s) on 1 MI355X, % of peak",
        "value": head["GB/s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len, "hq": w.hq,
                   "hkv": w.hkv, "head_dim": w.d, "sum_kv": sum(w.lens_kv),
                   "num_splits": w.num_splits, "plan": head["plan"],
                   "slot_plan": head["slot_plan"], "seed": w.seed,
                   "parallelism": "single-gpu"},
        "frac_of_hbm_peak": head["frac_of_hbm_peak"],
        "ms_per_step_min": head["ms_min"],
        "ms_per_step_mean": head["ms_mean"],
        "timing": "median of the timed steps (min and mean beside it), HIP events on the "
                  "library's stream, a 512 MiB cache flush before each step",
        "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if not args.no_others:
        _say("peaks")
        line["peaks"] = peaks(w, S, W, flush)
        del w
        torch.cuda.empty_cache()
        others = {}
        _say("spec_decode_planner")
        d5 = wl.make("spec_decode", device="cuda")
        d5.num_splits = 0
        others["spec_decode_planner"] = decode_line(sa, d5, S, W, flush, cpu_line)
        del d5
        torch.cuda.empty_cache()
        other_decode = "decode_gptoss" if args.workload == "spec_decode" else "spec_decode"
        _say(other_decode)
        others[other_decode] = decode_line(sa, wl.make(other_decode, device="cuda"), S, W, flush,
                                           cpu_line)
        torch.cuda.empty_cache()
        for name in ("varlen_prefill", "long_prefill"):
            _say(name)
            others[name] = prefill_line(sa, wl.make(name, device="cuda"), S, W, flush, cpu_line)
            torch.cuda.empty_cache()
        _say("chunked_prefill")
        p = wl.make("chunked_prefill", device="cuda")
        others["chunked_prefill"] = prefill_line(sa, p, S, W, flush, cpu_line, num_splits=0)
        r1 = prefill_line(sa, p, S, W, flush, 0, num_splits=1)
        others["chunked_prefill"]["unsplit_TFLOP/s"] = r1["TFLOP/s"]
        others["chunked_prefill"]["workload"] = "1024 new tokens over a 31744-token cached prefix"
        del p
        torch.cuda.empty_cache()
        _say("tiny_prefill")
        others["tiny_prefill"] = tiny_line(sa, S, W, flush, cpu_line)
        _say("paged decode / kv append")
        others.update(paged_lines(sa, S, W, flush, cpu_line))
        torch.cuda.empty_cache()
        line["others"] = others
    line["host"] = HOST
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
