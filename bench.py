"""Throughput of sink-aware GQA attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step is one pass of the whole decode hot path (split-KV kernel + log-sum-exp
merge of its partial slots) over the gpt-oss-like decode batch (64 sequences, 1 query token, Hq 64 over
Hkv 8, head_dim 64, KV lengths uniform in [1024, 8192]), with inputs resident in HBM.
Before every step a 512 MiB read (a sum over a scratch buffer) evicts the 256 MB
Infinity Cache and the L2s with clean lines, so each step streams its K/V from HBM and
pays no write-back of dirty lines; only the attention kernels sit inside the timed
event pair.  The line also reports the other workloads (varlen, long and chunked prefill
in TFLOP/s; speculative decode, decode over a paged cache and the paged KV append in
GB/s) and the fp64 CPU oracle on a bounded sample.

Algorithmic work (implementation overheads such as split partials are not counted):
  decode bytes  = K+V of every visible key once per KV head + Q + out + lse + sinks +
                  kv_indptr;  split kernel bytes = the same minus out and lse.
  prefill flops = 4 * head_dim * Hq * (visible query-key pairs).
"""
from __future__ import annotations

import argparse
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


def _say(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _pairs(lens_q, lens_kv, causal):
    tot = 0
    for lq, lk in zip(lens_q, lens_kv):
        if not causal:
            tot += lq * lk
            continue
        i = np.arange(lq, dtype=np.int64)
        tot += int(np.clip(i + lk - lq + 1, 0, lk).sum())
    return tot


def decode_bytes(w, split_only=False):
    kv = sum(w.lens_kv) * w.hkv * w.d * 2 * 2
    q = w.q.numel() * 2
    small = w.hq * 4 + (w.batch + 1) * 4
    if split_only:
        return kv + q + small
    return kv + q + q + w.batch * w.q_len * w.hq * 4 + small


def prefill_flops(w):
    return 4 * w.d * w.hq * _pairs(w.lens_q, w.lens_kv, w.causal)


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, n):
        self.ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]

    def mark(self, i, j):
        self.ev[i][j].record(torch.cuda.current_stream())

    def ms(self, j0, j1):
        return [e[j0].elapsed_time(e[j1]) for e in self.ev]


def _source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gqa_attention_sink_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def _traffic_for(kernel, workload):
    """HBM traffic measured by rocprofv3 counters for this kernel and workload, if the
    committed measurement was taken on the current kernel sources (else None)."""
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


def _c_call(fn, args):
    """One pre-marshalled C-ABI call (no Python argument handling between the events)."""
    rc = fn(*args)
    if rc != 0:
        raise RuntimeError(f"{fn.__name__} failed with status {rc}")


def bench_decode(sa, w, steps, warmup, flush):
    """Mean event times of the whole decode call and of its two kernels alone (the same
    launches decode makes).  The C entry points are called with arguments marshalled
    once, so no Python work separates an event from its kernel launch."""
    from gqa_attention_sink_amd import sink_attn as sam
    lib = sam.load()
    P = sam._ptr
    st = sam._stream(w.q.device)
    ws = sa.decode_workspace(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, w.num_splits)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.q_len, w.hq), dtype=torch.float32, device="cuda")
    s = sa.decode_num_slots(w.q_len, w.hq, w.hkv, w.d, w.max_kv, w.num_splits)
    rows = w.batch * w.q_len * w.hq
    tk = w.k.shape[1]
    scale, causal, ns, mk = float(w.scale), int(bool(w.causal)), int(w.num_splits), int(w.max_kv)
    stream = (sa.decode_stream_plan(w.batch, w.q_len, w.hq, w.hkv, w.d, tk, w.max_kv)
              if w.num_splits == 0 else None)
    full = (lib.sink_attn_decode, (P(w.q), P(w.k), P(w.v), P(w.sinks), P(w.cu_seqlens_kv),
                                   w.batch, w.q_len, tk, mk, w.hq, w.hkv, w.d, scale, causal, ns,
                                   P(ws), ws.numel(), P(out), P(lse), None, st))
    if stream is not None:  # the stream plan's two kernels, as decode runs them
        part = (lib.sink_attn_decode_stream_partial,
                (P(w.q), P(w.k), P(w.v), P(w.cu_seqlens_kv), w.batch, w.q_len, tk, mk, w.hq,
                 w.hkv, w.d, scale, causal, P(ws), ws.numel(), None, st))
        merge = (lib.sink_attn_decode_stream_merge,
                 (P(w.sinks), P(w.cu_seqlens_kv), w.batch, w.q_len, tk, mk, w.hq, w.hkv, w.d,
                  P(ws), ws.numel(), P(out), P(lse), st))
        po = pl = None
    else:
        po = torch.empty((rows, s, w.d), dtype=torch.float32, device="cuda")
        pl = torch.empty((rows, s), dtype=torch.float32, device="cuda")
        part = (lib.sink_attn_decode_partial,
                (P(w.q), P(w.k), P(w.v), P(w.sinks), P(w.cu_seqlens_kv), w.batch, w.q_len, tk,
                 mk, w.hq, w.hkv, w.d, scale, causal, ns, P(po), P(pl), None, st))
        merge = (lib.sink_attn_merge, (P(po), P(pl), rows, s, w.d, P(out), P(lse), st))

    def step_full(t=None, i=0):
        flush.sum()
        if t: t.mark(i, 0)
        _c_call(*full)
        if t: t.mark(i, 1)

    def step_split(t, i):
        flush.sum()
        t.mark(i, 0)
        _c_call(*part)
        t.mark(i, 1)
        _c_call(*merge)
        t.mark(i, 2)

    for _ in range(warmup):
        step_full()
    torch.cuda.synchronize()
    t = Timer(steps)
    t0 = time.perf_counter()
    for i in range(steps):
        step_full(t, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    full_ms = t.ms(0, 1)
    # the two kernels on their own (same launches as inside decode)
    t2 = Timer(steps)
    for i in range(steps):
        step_split(t2, i)
    torch.cuda.synchronize()
    split_ms = t2.ms(0, 1)
    merge_ms = t2.ms(1, 2)
    return dict(full_ms=float(np.mean(full_ms)), full_ms_min=float(np.min(full_ms)),
                split_ms=float(np.mean(split_ms)), merge_ms=float(np.mean(merge_ms)),
                wall_s=wall, slots=stream[2] if stream is not None else s,
                plan=("stream" if stream is not None else "chunks"),
                stream_plan=(dict(range_tokens=stream[0], ranges_per_head=stream[1],
                                  slots=stream[2]) if stream is not None else None))


def bench_prefill(sa, w, steps, warmup, flush, num_splits=1):
    out = torch.empty_like(w.q)
    lse = torch.empty((w.q.shape[0], w.hq), dtype=torch.float32, device="cuda")
    ws = None
    if num_splits != 1:
        ns = sa.prefill_num_splits(w.batch, w.max_q, w.max_kv, w.hq, w.hkv, num_splits)
        ws = torch.empty(max(256, sa.prefill_workspace_bytes(w.q.shape[0], w.hq, w.d, ns)),
                         dtype=torch.uint8, device="cuda")

    # pre-marshalled C call (no Python argument handling between the events)
    from gqa_attention_sink_amd import sink_attn as sam
    lib = sam.load()
    P = sam._ptr
    st = sam._stream(w.q.device)
    tq, tk = w.q.shape[0], w.k.shape[1]
    common = (P(w.q), P(w.k), P(w.v), P(w.sinks), P(w.cu_seqlens_q), P(w.cu_seqlens_kv),
              w.batch, int(w.max_q))
    tail = (tq, tk, w.hq, w.hkv, w.d, float(w.scale), int(bool(w.causal)))
    if num_splits == 1:
        call = (lib.sink_attn_prefill, common + tail + (P(out), P(lse), None, st))
    else:
        call = (lib.sink_attn_prefill_split,
                common + (int(w.max_kv),) + tail + (int(num_splits), P(ws), ws.numel(), P(out),
                                                    P(lse), None, st))

    def step(t=None, i=0):
        flush.sum()
        if t: t.mark(i, 0)
        _c_call(*call)
        if t: t.mark(i, 1)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t = Timer(steps)
    t0 = time.perf_counter()
    for i in range(steps):
        step(t, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = t.ms(0, 1)
    return dict(ms=float(np.mean(ms)), ms_min=float(np.min(ms)), wall_s=wall)


# YaRN parameters of the rotated bench lines (a long-context configuration: 32x over a
# 4096-token original context)
YARN_BENCH = dict(theta=150000.0, factor=32.0, original_max_pos=4096, beta_fast=32.0,
                  beta_slow=1.0)


def time_calls(fn, steps, warmup, flush):
    """Mean/min milliseconds of fn() between HIP events, each call after a cache flush."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t = Timer(steps)
    for i in range(steps):
        flush.sum()
        t.mark(i, 0)
        fn()
        t.mark(i, 1)
    torch.cuda.synchronize()
    ms = t.ms(0, 1)
    return float(np.mean(ms)), float(np.min(ms))


def bench_paged(sa, steps, warmup, flush):
    """Decode over a paged cache (the gpt-oss-like batch, page_size 16, pages scattered
    by a seeded permutation) and the KV append of a mixed-length prefill batch into a
    paged cache.  Bytes are algorithmic: decode as the contiguous decode plus the page
    list; append = new K and V read once and written once."""
    from gqa_attention_sink_amd import workloads as wl
    res = {}
    w = wl.make("decode_gptoss", device="cuda")
    pk = wl.make_paged(w, 16, seed=4242)
    ws = sa.decode_workspace(w.batch, w.q_len, w.hq, w.hkv, w.d, w.max_kv, w.num_splits)
    out = torch.empty_like(w.q)
    lse = torch.empty((w.batch, w.q_len, w.hq), dtype=torch.float32, device="cuda")
    fn = lambda: sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,  # noqa: E731
                                 pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale,
                                 w.causal, w.num_splits, workspace=ws, out=out, lse=lse)
    ms, ms_min = time_calls(fn, steps, warmup, flush)
    nbytes = decode_bytes(w) + pk.kv_page_indices.numel() * 4 + w.batch * 4
    res["paged_decode"] = {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2),
                           "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "ms": round(ms, 4), "ms_min": round(ms_min, 4), "page_size": 16,
                           "workload": "decode_gptoss in a paged cache", "bytes": nbytes}
    # the same step with the queries rotated (YaRN) as the kernel loads them
    rope = sa.RopeParams(**YARN_BENCH)
    fn = lambda: sa.decode_paged(w.q, pk.k_cache, pk.v_cache, w.sinks, pk.kv_page_indptr,  # noqa: E731
                                 pk.kv_page_indices, pk.kv_last_page_len, w.max_kv, w.scale,
                                 w.causal, w.num_splits, workspace=ws, out=out, lse=lse,
                                 rope=rope)
    ms, ms_min = time_calls(fn, steps, warmup, flush)
    res["paged_decode_rope"] = {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2),
                                "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                "ms": round(ms, 4), "ms_min": round(ms_min, 4),
                                "workload": "paged_decode with fused YaRN rotation of q",
                                "rope": YARN_BENCH}
    del pk, ws
    torch.cuda.empty_cache()
    p = wl.make("varlen_prefill", device="cuda")
    pk = wl.make_paged(p, 16, seed=4343)
    k_new = p.k.permute(1, 0, 2).contiguous()
    v_new = p.v.permute(1, 0, 2).contiguous()
    app = p.cu_seqlens_kv
    fn = lambda: sa.kv_append(k_new, v_new, app, pk.kv_page_indptr, pk.kv_page_indices,  # noqa: E731
                              pk.kv_last_page_len, pk.k_cache, pk.v_cache, p.max_kv)
    ms, ms_min = time_calls(fn, steps, warmup, flush)
    nbytes = 2 * 2 * k_new.numel() * 2
    res["kv_append"] = {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2),
                        "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "ms": round(ms, 4), "ms_min": round(ms_min, 4), "page_size": 16,
                        "workload": "varlen_prefill K/V appended to a paged cache",
                        "tokens": int(k_new.shape[0]), "bytes": nbytes}
    fn = lambda: sa.kv_append(k_new, v_new, app, pk.kv_page_indptr, pk.kv_page_indices,  # noqa: E731
                              pk.kv_last_page_len, pk.k_cache, pk.v_cache, p.max_kv, rope=rope)
    ms, ms_min = time_calls(fn, steps, warmup, flush)
    res["kv_append_rope"] = {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2),
                             "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "ms": round(ms, 4), "ms_min": round(ms_min, 4),
                             "workload": "kv_append with fused YaRN rotation of the keys"}
    return res


def cpu_baseline(w_gpu, budget_s=20.0):
    """The fp64 oracle on a bounded sample of the decode workload: whole sequences,
    taken in order until about budget_s seconds of CPU work; the rate is scaled to the
    metric's unit (algorithmic GB/s of the sample)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    ind = w_gpu.cu_seqlens_kv.cpu().tolist()
    done_bytes, t_used, nseq = 0, 0.0, 0
    for b in range(w_gpu.batch):
        ks = slice(ind[b], ind[b + 1])
        q = w_gpu.q[b:b + 1].cpu()
        k = w_gpu.k[:, ks].cpu()
        v = w_gpu.v[:, ks].cpu()
        t0 = time.perf_counter()
        oracle.sink_attention_decode(q, k, v, w_gpu.sinks, [0, ind[b + 1] - ind[b]],
                                     w_gpu.scale, w_gpu.causal)
        t_used += time.perf_counter() - t0
        lk = ind[b + 1] - ind[b]
        done_bytes += lk * w_gpu.hkv * w_gpu.d * 4 + 2 * q.numel() * 2 + w_gpu.q_len * w_gpu.hq * 4
        nseq += 1
        if t_used >= budget_s:
            break
    return {"value": round(done_bytes / t_used / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{nseq} of {w_gpu.batch} sequences of {w_gpu.name} (all heads), "
                      f"{t_used:.1f} s of fp64 numpy on the host"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_gptoss")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the reference "
                         "kernel for scaling HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
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
    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    _say(f"workload {args.workload}")
    w = wl.make(args.workload, device="cuda")
    assert w.kind == "decode", "the headline step is the decode path"
    r = bench_decode(sa, w, args.steps, args.warmup, flush)
    nbytes = decode_bytes(w)
    split_bytes = decode_bytes(w, split_only=True)
    value = nbytes / (r["full_ms"] * 1e-3) / 1e9
    split_gbs = split_bytes / (r["split_ms"] * 1e-3) / 1e9
    # the dominant kernel: the stream kernel under the stream plan, else the chunk-wave
    # kernel when a workgroup merges several chunks, else the split kernel
    if r["plan"] == "stream":
        kname = "decode_stream_kernel"
    elif sa.decode_chunks_per_slot(w.q_len, w.hq, w.hkv, w.d) > 1:
        kname = "decode_cw_kernel"
    else:
        kname = "decode_split_kernel"
    line = {
        "metric": "sink-attn decode HBM GB/s (and prefill TFLOP/s) on 1 MI355X, % of peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["full_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len, "hq": w.hq,
                   "hkv": w.hkv, "head_dim": w.d, "sum_kv": sum(w.lens_kv),
                   "num_splits": w.num_splits, "plan": r["plan"], "slots": r["slots"],
                   "stream_plan": r["stream_plan"], "seed": w.seed,
                   "parallelism": "single-gpu"},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "ms_per_step_min": round(r["full_ms_min"], 4),
        "wall_ms_per_step_incl_flush": round(r["wall_s"] * 1e3 / args.steps, 4),
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(split_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(split_gbs / HBM_PEAK_GBS, 4),
                     "traffic": _traffic_for(kname, w.name),
                     "algorithmic_bytes_per_launch": split_bytes,
                     "avg_launch_ms": round(r["split_ms"], 4),
                     "merge_ms": round(r["merge_ms"], 4)},
    }
    others = {}
    if not args.no_others:
        del w
        torch.cuda.empty_cache()
        for name in ("varlen_prefill", "long_prefill"):
            _say(f"workload {name}")
            p = wl.make(name, device="cuda")
            rp = bench_prefill(sa, p, args.steps, args.warmup, flush)
            fl = prefill_flops(p)
            tf = fl / (rp["ms"] * 1e-3) / 1e12
            others[name] = {"TFLOP/s": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                            "ms": round(rp["ms"], 4), "ms_min": round(rp["ms_min"], 4),
                            "flops": fl}
            del p
            torch.cuda.empty_cache()
        _say("workload chunked_prefill")
        p = wl.make("chunked_prefill", device="cuda")
        fl = prefill_flops(p)
        ns = sa.prefill_num_splits(p.batch, p.max_q, p.max_kv, p.hq, p.hkv, 0)
        rs = bench_prefill(sa, p, args.steps, args.warmup, flush, num_splits=0)
        r1 = bench_prefill(sa, p, args.steps, args.warmup, flush, num_splits=1)
        tf = fl / (rs["ms"] * 1e-3) / 1e12
        others["chunked_prefill"] = {
            "TFLOP/s": round(tf, 2), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
            "ms": round(rs["ms"], 4), "ms_min": round(rs["ms_min"], 4), "flops": fl,
            "key_splits": ns, "unsplit_TFLOP/s": round(fl / (r1["ms"] * 1e-3) / 1e12, 2),
            "workload": "1024 new tokens over a 31744-token cached prefix"}
        del p
        torch.cuda.empty_cache()
        _say("workload spec_decode")
        d5 = wl.make("spec_decode", device="cuda")
        r5 = bench_decode(sa, d5, max(5, args.steps // 2), 2, flush)
        b5 = decode_bytes(d5)
        g5 = b5 / (r5["full_ms"] * 1e-3) / 1e9
        s5 = decode_bytes(d5, True) / (r5["split_ms"] * 1e-3) / 1e9
        others["spec_decode"] = {"GB/s": round(g5, 2), "frac_of_hbm_peak": round(g5 / HBM_PEAK_GBS, 4),
                                 "ms": round(r5["full_ms"], 4), "split_kernel_GB/s": round(s5, 2),
                                 "split_ms": round(r5["split_ms"], 4),
                                 "merge_ms": round(r5["merge_ms"], 4), "bytes": b5,
                                 "plan": "32 chunks per sequence (as the workload names)"}
        # the same batch under the planner (num_splits = 0): the stream plan
        d5.num_splits = 0
        r6 = bench_decode(sa, d5, max(5, args.steps // 2), 2, flush)
        g6 = b5 / (r6["full_ms"] * 1e-3) / 1e9
        s6 = decode_bytes(d5, True) / (r6["split_ms"] * 1e-3) / 1e9
        others["spec_decode_planner"] = {
            "GB/s": round(g6, 2), "frac_of_hbm_peak": round(g6 / HBM_PEAK_GBS, 4),
            "ms": round(r6["full_ms"], 4), "split_kernel_GB/s": round(s6, 2),
            "split_ms": round(r6["split_ms"], 4), "merge_ms": round(r6["merge_ms"], 4),
            "bytes": b5, "plan": r6["plan"], "stream_plan": r6["stream_plan"]}
        del d5
        torch.cuda.empty_cache()
        _say("workload paged decode / kv append")
        others.update(bench_paged(sa, max(5, args.steps // 2), 2, flush))
        torch.cuda.empty_cache()
        line["others"] = others
    if not args.no_cpu_baseline:
        _say("cpu baseline (oracle)")
        w = wl.make(args.workload, device="cuda")
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
