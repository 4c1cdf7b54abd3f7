"""C-ABI checks that need no GPU: the library loads, exports every entry point that
include/sink_attn.h declares, and rejects every invalid argument the host can see
before making any HIP call."""
import ctypes
import math
import os
import re
import subprocess

import pytest

from gqa_attention_sink_amd import sink_attn as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sink_attn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation
# or has nothing to compute, so none of them launches a kernel


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sa.LIB_PATH):
        from gqa_attention_sink_amd.build import build
        build()
    return sa.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\*?\s+\*?(sink_attn_[a-z_0-9]+)\(",
                                 text, flags=re.M)))


def test_header_declares_entry_points():
    names = _declared()
    for n in ("sink_attn_prefill", "sink_attn_decode", "sink_attn_decode_workspace_bytes",
              "sink_attn_merge", "sink_attn_status_str", "sink_attn_decode_partial",
              "sink_attn_decode_num_slots", "sink_attn_decode_chunks_per_slot"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", sa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(ln.split()[-1] for ln in out.splitlines() if ln.strip())
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        assert hasattr(lib, n)


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=None, cq=FAKE, ck=FAKE, batch=1, maxq=16, tq=16,
             tk=16, hq=8, hkv=2, d=64, scale=0.125, causal=1, out=FAKE, lse=None)
    a.update(kw)
    return lib.sink_attn_prefill(a["q"], a["k"], a["v"], a["sinks"], a["cq"], a["ck"],
                                 a["batch"], a["maxq"], a["tq"], a["tk"], a["hq"], a["hkv"],
                                 a["d"], a["scale"], a["causal"], a["out"], a["lse"], None, None)


def _decode(lib, **kw):
    # 32 rows per KV head: one chunk per wavefront, 4 slots, so a workspace is needed
    a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=None, ind=FAKE, batch=2, ql=1, tk=64, maxk=32,
             hq=64, hkv=2, d=64, scale=0.125, causal=1, ns=0, ws=None, wsb=0, out=FAKE, lse=None)
    a.update(kw)
    return lib.sink_attn_decode(a["q"], a["k"], a["v"], a["sinks"], a["ind"], a["batch"],
                                a["ql"], a["tk"], a["maxk"], a["hq"], a["hkv"], a["d"],
                                a["scale"], a["causal"], a["ns"], a["ws"], a["wsb"], a["out"],
                                a["lse"], None, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(cq=None), INVALID), (dict(ck=None), INVALID), (dict(out=None), INVALID),
    (dict(batch=0), INVALID), (dict(hq=6, hkv=4), INVALID), (dict(hkv=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(causal=2), INVALID), (dict(maxq=-1), INVALID), (dict(tq=-5), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(d=0), UNSUPPORTED),
    (dict(maxq=0), OK), (dict(tq=0), OK),
])
def test_prefill_validation(lib, kw, rc):
    assert _prefill(lib, **kw) == rc


@pytest.mark.parametrize("kw,rc", [
    (dict(q=None), INVALID), (dict(ind=None), INVALID), (dict(out=None), INVALID),
    (dict(hq=8, hkv=3), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(ns=-1), INVALID), (dict(ns=65), INVALID), (dict(batch=0), INVALID),
    (dict(causal=-1), INVALID), (dict(maxk=-3), INVALID),
    (dict(ql=0), UNSUPPORTED), (dict(ql=5), UNSUPPORTED), (dict(d=80), UNSUPPORTED),
    (dict(maxk=1 << 24, d=128), UNSUPPORTED),
    (dict(ws=None, wsb=0), WORKSPACE), (dict(ws=FAKE, wsb=16), WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x1010), wsb=1 << 30), WORKSPACE),  # misaligned
])
def test_decode_validation(lib, kw, rc):
    assert _decode(lib, **kw) == rc


def test_decode_partial_validation(lib):
    f = lib.sink_attn_decode_partial
    assert f(FAKE, FAKE, FAKE, None, FAKE, 2, 1, 64, 32, 8, 2, 64, 0.125, 1, 0, None, FAKE, None, None) == INVALID
    assert f(FAKE, FAKE, FAKE, None, FAKE, 2, 9, 64, 32, 8, 2, 64, 0.125, 1, 0, FAKE, FAKE, None, None) == UNSUPPORTED


def test_merge_validation(lib):
    m = lib.sink_attn_merge
    assert m(None, FAKE, None, 4, 2, 64, FAKE, None, None) == INVALID
    assert m(FAKE, FAKE, None, 4, 0, 64, FAKE, None, None) == INVALID
    assert m(FAKE, FAKE, FAKE, 4, 257, 64, FAKE, None, None) == INVALID
    assert m(FAKE, FAKE, None, -1, 2, 64, FAKE, None, None) == INVALID
    assert m(FAKE, FAKE, None, 4, 2, 72, FAKE, None, None) == UNSUPPORTED
    assert m(FAKE, FAKE, None, 0, 2, 64, FAKE, None, None) == OK
    assert m(FAKE, FAKE, FAKE, 0, 2, 64, FAKE, None, None) == OK


def test_planner_slots(lib):
    def ns(ql, hq, hkv, d, maxk, splits, batch=1, cus=256):
        return lib.sink_attn_decode_num_slots(batch, ql, hq, hkv, d, maxk, splits, cus)
    def cps(ql, hq, hkv, d, maxk=1024, splits=0, batch=1, cus=256):
        return lib.sink_attn_decode_chunks_per_slot(batch, ql, hq, hkv, d, maxk, splits, cus)
    # planner mode, more than 16 rows per KV head (here 4 x 8 = 32): one chunk per slot
    assert cps(4, 32, 4, 64) == 1
    assert ns(4, 32, 4, 64, 8192, 0) == 16 and ns(4, 32, 4, 64, 1024, 0) == 4
    assert ns(4, 32, 4, 64, 100, 0) == 4 and ns(4, 32, 4, 64, 0, 0) == 4
    assert ns(4, 32, 4, 64, 2049, 0) == 9 and ns(4, 32, 4, 64, 100000, 0) == 16
    assert ns(4, 32, 4, 64, 10, 1) == 1
    # forced chunks, more than 16 rows: runs of chunks, as long as about four workgroups
    # per CU remain.  Speculative decode (256 x 4 KV heads, 32 chunks): 32768 chunk
    # workgroups / 1024 -> runs of 32, one slot; a single sequence: runs of 1
    assert cps(4, 64, 4, 128, 32768, 32, batch=256) == 32
    assert ns(4, 64, 4, 128, 32768, 32, batch=256) == 1
    assert cps(4, 64, 4, 128, 32768, 32, batch=1) == 1 and ns(4, 64, 4, 128, 32768, 32) == 32
    assert cps(4, 64, 4, 128, 32768, 32, batch=64) == 8          # 8192 / 1024
    assert ns(4, 64, 4, 128, 32768, 32, batch=64) == 4
    assert cps(4, 64, 4, 128, 32768, 32, batch=64, cus=80) == 25  # 8192 / 320
    assert ns(4, 64, 4, 128, 32768, 32, batch=64, cus=80) == 2
    assert cps(4, 64, 2, 128, 32768, 7, batch=300) == 7           # rows 128: 2 row groups
    # <= 16 rows: 4 chunks per slot (head_dim 64) or 2 (head_dim 128); the planner rounds
    # ceil(Lk/256) up to a multiple of that before clamping to [4, 16]
    assert cps(1, 64, 8, 64) == 4 and cps(1, 64, 8, 128) == 2 and cps(2, 16, 2, 64) == 4
    assert cps(1, 64, 8, 64, 32768, 32, batch=500) == 4          # forced: same grouping
    assert ns(1, 64, 8, 64, 8192, 0) == 4 and ns(1, 64, 8, 64, 1024, 0) == 1
    assert ns(1, 64, 8, 64, 1025, 0) == 2 and ns(1, 64, 8, 64, 3000, 0) == 3
    assert ns(1, 64, 8, 128, 2049, 0) == 5 and ns(1, 64, 8, 128, 100, 0) == 2
    assert ns(1, 64, 8, 64, 32768, 7) == 2 and ns(1, 64, 8, 64, 10, 1) == 1
    # invalid arguments
    assert ns(1, 64, 8, 64, 10, 65) == 0 and ns(1, 64, 8, 64, -1, 0) == 0
    assert ns(0, 64, 8, 64, 10, 0) == 0 and ns(1, 64, 7, 64, 10, 0) == 0
    assert ns(1, 64, 8, 96, 10, 0) == 0 and cps(5, 64, 8, 64) == 0
    assert ns(1, 64, 8, 64, 10, 0, batch=0) == 0 and ns(1, 64, 8, 64, 10, 0, cus=-1) == 0


def test_workspace_bytes(lib):
    wb = lib.sink_attn_decode_workspace_bytes
    # speculative decode, 32 chunks: runs of 32 chunks per workgroup on 256 CUs (the
    # planned-for count with no device), so one slot
    rows, s, d = 256 * 4 * 64, 1, 128
    o = rows * s * d * 4
    o = (o + 255) // 256 * 256
    expect = (o + rows * s * 4 + 255) // 256 * 256
    assert wb(256, 4, 64, 4, 128, 32768, 32) == expect
    rows, s, d = 64 * 64, 4, 64                      # 16 planned chunks in 4 slots
    o = (rows * s * d * 4 + 255) // 256 * 256
    assert wb(64, 1, 64, 8, 64, 8192, 16) == (o + rows * s * 4 + 255) // 256 * 256
    # planner mode with <= 16 rows per KV head may take the stream plan: 17 slots
    s = 17
    o = (rows * s * d * 4 + 255) // 256 * 256
    assert wb(64, 1, 64, 8, 64, 8192, 0) == (o + rows * s * 4 + 255) // 256 * 256
    # 128 rows per KV head (chunk plan only, one chunk per slot): 16 slots
    rows, s = 64 * 4 * 64, 16
    o = (rows * s * d * 4 + 255) // 256 * 256
    assert wb(64, 4, 64, 2, 64, 8192, 0) == (o + rows * s * 4 + 255) // 256 * 256
    assert wb(0, 1, 8, 8, 64, 10, 0) == 0 and wb(1, 5, 8, 8, 64, 10, 0) == 0
    assert wb(1, 1, 8, 8, 96, 10, 0) == 0 and wb(1, 1, 8, 3, 64, 10, 0) == 0


def test_status_strings(lib):
    for rc in range(7):
        assert lib.sink_attn_status_str(rc).decode().startswith("SINK_ATTN_")
    assert b"unknown" in lib.sink_attn_status_str(99)
    assert re.match(rb"\d+\.\d+\.\d+", lib.sink_attn_version())


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        sa.prefill(q, k, k, None, cu, cu, 4)


def test_paged_validation(lib):
    dp = lib.sink_attn_decode_paged
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, sinks=None, ind=FAKE, idx=FAKE, last=FAKE, batch=2,
                 ql=1, ent=8, pages=8, ps=16, maxk=32, hq=64, hkv=2, d=64, scale=0.125,
                 causal=1, ns=0, ws=None, wsb=0, out=FAKE, lse=None)
        a.update(kw)
        return dp(a["q"], a["k"], a["v"], a["sinks"], a["ind"], a["idx"], a["last"], a["batch"],
                  a["ql"], a["ent"], a["pages"], a["ps"], a["maxk"], a["hq"], a["hkv"], a["d"],
                  a["scale"], a["causal"], a["ns"], a["ws"], a["wsb"], a["out"], a["lse"], None, None)
    assert call(idx=None) == INVALID and call(last=None) == INVALID and call(ind=None) == INVALID
    assert call(pages=0) == INVALID and call(ent=-1) == INVALID
    assert call(ps=8) == UNSUPPORTED and call(ps=24) == UNSUPPORTED and call(ps=8192) == UNSUPPORTED
    assert call(hq=64, hkv=3) == INVALID and call(d=96) == UNSUPPORTED and call(ql=5) == UNSUPPORTED
    assert call(ws=None, wsb=0) == WORKSPACE   # 32 rows per KV head: 4 slots need a workspace
    ap = lib.sink_attn_kv_append
    def acall(**kw):
        a = dict(kn=FAKE, vn=FAKE, app=FAKE, ind=FAKE, idx=FAKE, last=FAKE, batch=2, maxn=4,
                 tot=8, ent=8, pages=8, ps=16, hkv=2, d=64, kc=FAKE, vc=FAKE)
        a.update(kw)
        return ap(a["kn"], a["vn"], a["app"], a["ind"], a["idx"], a["last"], a["batch"], a["maxn"],
                  a["tot"], a["ent"], a["pages"], a["ps"], a["hkv"], a["d"], a["kc"], a["vc"],
                  a.get("rope"), None)
    assert acall(kn=None) == INVALID and acall(kc=None) == INVALID and acall(app=None) == INVALID
    assert acall(batch=0) == INVALID and acall(pages=0) == INVALID and acall(hkv=0) == INVALID
    assert acall(ps=20) == UNSUPPORTED and acall(d=80) == UNSUPPORTED
    assert acall(maxn=0) == OK and acall(tot=0) == OK      # nothing to write: no launch


def test_rope_validation(lib):
    R = sa.RopeParams
    ra = lib.sink_attn_rope_apply
    ok = R(150000.0, 32.0, 4096, 32.0, 1.0)
    import ctypes as C
    def call(rope, **kw):
        a = dict(x=FAKE, n=4, h=2, d=64, ts=128, hs=64, pos=FAKE)
        a.update(kw)
        return ra(a["x"], a["n"], a["h"], a["d"], a["ts"], a["hs"], a["pos"],
                  None if rope is None else C.byref(rope), None)
    assert call(None) == INVALID                            # rope required here
    assert call(R(1.0)) == INVALID and call(R(-5.0)) == INVALID
    assert call(R(10000.0, 0.0)) == INVALID and call(R(float("nan"))) == INVALID
    assert call(R(10000.0, 4.0, 0)) == INVALID               # YaRN needs the original length
    assert call(R(10000.0, 4.0, 4096, 1.0, 1.0)) == INVALID  # beta_fast must exceed beta_slow
    assert call(ok, d=96) == UNSUPPORTED and call(ok, ts=100) == INVALID
    assert call(ok, x=C.c_void_p(0x1008)) == INVALID          # 16-byte alignment
    assert call(ok, n=0) == OK                                # nothing to rotate: no launch
    # a bad rope on an attention entry point is rejected before any launch
    bad = C.byref(R(1.0))
    assert lib.sink_attn_prefill(FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 16, 16, 16, 8, 2, 64,
                                 0.125, 1, FAKE, None, bad, None) == INVALID


def test_prefill_split_planner_and_validation(lib):
    def ns(*a):
        return lib.sink_attn_prefill_num_splits(*a, 256)   # planned for 256 CUs
    # 1024 new tokens over 32768 keys, 64 query heads over 8: 16 head groups (4 heads each)
    # x 16 query tiles (64 positions) = 256 workgroups -> 4 splits for ~1024
    assert ns(1, 1024, 32768, 64, 8, 0) == 4
    assert ns(2, 2048, 32768, 64, 8, 0) == 1          # 1024 workgroups already
    assert ns(1, 64, 32768, 64, 8, 0) == 16           # tiny grid: capped at 16
    assert ns(1, 64, 1024, 64, 8, 0) == 2             # at least 512 keys per split
    assert ns(1, 6000, 6000, 64, 4, 0) == 1           # a full prefill fills the GPU
    assert ns(1, 64, 100, 64, 8, 0) == 1 and ns(2, 64, 64, 8, 8, 5) == 5
    assert ns(0, 1, 1, 8, 8, 0) == 0 and ns(1, 1, 1, 8, 3, 0) == 0 and ns(1, 1, 1, 8, 8, 65) == 0
    assert lib.sink_attn_prefill_num_splits(1, 1, 1, 8, 8, 0, -1) == 0
    wb = lib.sink_attn_prefill_workspace_bytes
    rows, s, d = 4096 * 64, 4, 64
    o = (rows * s * d * 4 + 255) // 256 * 256
    assert wb(4096, 64, 64, 4) == (o + rows * s * 4 + 255) // 256 * 256
    assert wb(4096, 64, 64, 1) == 0 and wb(4096, 64, 96, 4) == 0
    f = lib.sink_attn_prefill_split
    def call(**kw):
        a = dict(ns=4, ws=None, wsb=0, maxkv=4096, d=64)
        a.update(kw)
        return f(FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, 256, a["maxkv"], 256, 4096, 64, 8, a["d"],
                 0.125, 1, a["ns"], a["ws"], a["wsb"], FAKE, None, None, None)
    assert call() == WORKSPACE                       # 4 splits need a workspace
    assert call(ns=-1) == INVALID and call(ns=65) == INVALID and call(maxkv=-1) == INVALID
    assert call(d=80) == UNSUPPORTED


# ---------------------------------------------------------------- plans sized by CUs
@pytest.mark.parametrize("cus", [256, 80, 32])
def test_prefill_splits_follow_cu_count(lib, cus):
    """About four 8-wavefront workgroups per CU: the chunked-prefill grid (256
    workgroups) is split until it reaches 4*cus, at most 16 splits of >= 512 keys."""
    ns = lib.sink_attn_prefill_num_splits
    base = 16 * 16                                     # head groups x query tiles
    want = min(16, max(1, -(-4 * cus // base)), 32768 // 64 // 8)
    assert ns(1, 1024, 32768, 64, 8, 0, cus) == want
    assert ns(1, 6000, 6000, 64, 4, 0, cus) == 1     # already >= 4 per CU
    assert ns(1, 1024, 32768, 64, 8, 3, cus) == 3    # forced


@pytest.mark.parametrize("cus", [256, 80, 32])
@pytest.mark.parametrize("b,ql,hq,hkv,d,total,maxkv,per_cu", [
    (64, 1, 64, 8, 64, 294802, 8192, 4),      # <= 16 rows: ~4 wavefronts per CU
    (256, 4, 64, 4, 128, 256 * 32768, 32768, 2),  # 64 rows: ~2 workgroups per CU
])
def test_stream_plan_follows_cu_count(lib, cus, b, ql, hq, hkv, d, total, maxkv, per_cu):
    r, n, s = (sa.ctypes.c_int32(), sa.ctypes.c_int32(), sa.ctypes.c_int32())
    ok = lib.sink_attn_decode_stream_plan(b, ql, hq, hkv, d, total, maxkv, cus,
                                          sa.ctypes.byref(r), sa.ctypes.byref(n),
                                          sa.ctypes.byref(s))
    assert ok == 1
    assert n.value == per_cu * cus // hkv               # ranges per KV head
    assert r.value % 32 == 0 and n.value * r.value >= total
    assert r.value >= -(-maxkv // 16) and s.value <= 17
    # fewer CUs: longer ranges, never more work units than the device holds at once
    assert n.value * hkv <= per_cu * cus
    assert lib.sink_attn_decode_stream_plan(b, ql, hq, hkv, d, total, maxkv, -1, None, None,
                                            None) == 0


@pytest.mark.parametrize("cus", [256, 80, 32])
def test_decode_plan_kind(lib, cus):
    """sink_attn_decode picks whole-sequence runs (2) in planner mode when there are more
    than 16 rows per KV head, at least two workgroups per CU and sequences of nearly
    equal length; else the stream plan (1) where it applies, else the chunk plan (0)."""
    kind = lib.sink_attn_decode_plan_kind
    spec = (4, 64, 4, 128)                    # 64 rows per KV head, one row group
    b = -(-2 * cus // 4)                      # the fewest sequences with 2 workgroups per CU
    assert kind(b, *spec, b * 32768, 32768, 0, cus) == 2
    assert kind(b - 1, *spec, (b - 1) * 32768, 32768, 0, cus) == 1     # under-filled
    t78 = -(-7 * b * 32768 // 8)              # total at exactly 7/8 of batch * max
    assert kind(b, *spec, t78, 32768, 0, cus) == 2
    assert kind(b, *spec, t78 - 1, 32768, 0, cus) == 1                 # unequal lengths
    assert kind(b, *spec, b * 32768, 32768, 32, cus) == 0              # forced chunks
    assert kind(b, *spec, 0, 0, 0, cus) == 1                           # no keys: no runs
    # 8 rows per KV head (the gpt-oss batch): never whole runs
    assert kind(4 * cus, 1, 64, 8, 64, 4 * cus * 4096, 4096, 0, cus) == 1
    # more than 64 rows per KV head (two row groups of 64): whole runs or chunks
    assert kind(cus, 4, 128, 4, 64, cus * 4096, 4096, 0, cus) == 2
    assert kind(cus // 8, 4, 128, 4, 64, cus // 8 * 4096, 4096, 0, cus) == 0
    # invalid sizes
    assert kind(0, *spec, 0, 0, 0, cus) == -1
    assert kind(b, *spec, b * 32768, 32768, 65, cus) == -1
    assert kind(b, *spec, b * 32768, 32768, 0, -1) == -1


# ---------------------------------------------------------------- decode chunk plan
def _bounds(lib, lk, ql, hq, hkv, d, ns):
    n = lib.sink_attn_decode_chunk_bounds(lk, ql, hq, hkv, d, ns, None, 0)
    buf = (sa.ctypes.c_int32 * (n + 1))()
    assert lib.sink_attn_decode_chunk_bounds(lk, ql, hq, hkv, d, ns, buf, n + 1) == n
    return list(buf)


@pytest.mark.parametrize("ql,hq,hkv,d", [(1, 64, 8, 64), (4, 64, 4, 128), (2, 16, 4, 64),
                                         (1, 64, 8, 128), (4, 32, 4, 64)])
def test_decode_chunk_plan_is_a_partition(lib, ql, hq, hkv, d):
    """The plan the kernels derive per sequence: a partition of [0, Lk) into equal
    32-key-aligned chunks (trailing ones may be empty); the planner picks 4..16 chunks,
    a multiple of the chunks one workgroup merges; a forced count is taken as given."""
    cps = lib.sink_attn_decode_chunks_per_slot(1, ql, hq, hkv, d, 1024, 0, 256)
    for lk in (0, 1, 31, 32, 33, 255, 256, 1000, 1024, 1025, 4097, 8192, 32768, 100000):
        for ns in (0, 1, 3, 7, 32, 64):
            b = _bounds(lib, lk, ql, hq, hkv, d, ns)
            n = len(b) - 1
            assert b[0] == 0 and b[-1] == lk and all(x <= y for x, y in zip(b, b[1:]))
            lens = [y - x for x, y in zip(b, b[1:])]
            # cuts inside the sequence sit on 32-key stage boundaries
            assert all(x % 32 == 0 for x in b[:-1] if x < lk)
            # non-empty chunks share one length (the last may be shorter), no longer than
            # 32-key alignment forces: (len - 32) * n < lk
            full = [x for x in lens if x > 0]
            if len(full) > 1:
                cl = full[0]
                assert cl % 32 == 0 and all(x == cl for x in full[:-1]) and full[-1] <= cl
                assert (cl - 32) * n < lk
            assert all(x == 0 for x in lens[len(full):])      # empty chunks trail
            if ns:
                assert n == ns
            else:
                assert 4 <= n <= 16 and n % cps == 0
                assert n >= min(16, -(-lk // 256))           # about 256 keys per chunk at most
    # the gpt-oss decode lengths (1024..8192 keys, 8 rows per KV head, 4 chunks merged per
    # workgroup) get 4..16 chunks, as that workload asks
    if (ql, hq, hkv, d) == (1, 64, 8, 64):
        for lk in (1024, 2048, 4096, 8192):
            n = len(_bounds(lib, lk, ql, hq, hkv, d, 0)) - 1
            assert 4 <= n <= 16
    # the speculative decode's 32 chunks of 1024 keys
    if (ql, hq, hkv, d) == (4, 64, 4, 128):
        assert _bounds(lib, lk=32768, ql=4, hq=64, hkv=4, d=128, ns=32) == list(range(0, 32769, 1024))


def test_decode_chunk_plan_rejects(lib):
    f = lib.sink_attn_decode_chunk_bounds
    assert f(-1, 1, 64, 8, 64, 0, None, 0) == 0 and f(10, 5, 64, 8, 64, 0, None, 0) == 0
    assert f(10, 1, 64, 8, 80, 0, None, 0) == 0 and f(10, 1, 64, 8, 64, 65, None, 0) == 0
    assert f(10, 1, 64, 8, 64, 0, None, 3) == 0       # capacity without a buffer
    buf = (sa.ctypes.c_int32 * 3)(-7, -7, -7)
    assert f(1000, 1, 64, 8, 64, 4, buf, 2) == 4      # only `capacity` entries written
    assert list(buf) == [0, 256, -7]


# ---------------------------------------------------------------- in-place rotation, append
def test_rope_apply_rejects_overlapping_rows(lib):
    R = sa.RopeParams
    ra = lib.sink_attn_rope_apply
    ok = sa.ctypes.byref(R(150000.0, 32.0, 4096, 32.0, 1.0))
    def call(n, h, d, ts, hs):
        return ra(FAKE, n, h, d, ts, hs, FAKE, ok, None)
    # token-major [T, H, D] and head-major [H, T, D] are accepted: they pass validation
    # and would launch (with no device that ends in a HIP error).  Never run with a
    # device: the pointers are fake.
    import torch
    if not torch.cuda.is_available():
        for args in ((4, 2, 64, 128, 64), (4, 2, 64, 64, 256), (1, 1, 64, 0, 0),
                     (4, 1, 64, 64, 0), (1, 3, 128, 0, 128)):
            assert call(*args) not in (INVALID, UNSUPPORTED), args
    # rows that overlap: rotated twice by racing lanes -> rejected
    for args in ((4, 2, 64, 0, 64), (4, 2, 64, 64, 0), (4, 2, 64, 32, 256), (1, 2, 64, 0, 32),
                 (3, 1, 64, 8, 0), (4, 2, 64, 64, 128), (4, 4, 64, 128, 64)):
        assert call(*args) == INVALID, args


def test_kv_append_rejects_misaligned(lib):
    ap = lib.sink_attn_kv_append
    odd = sa.ctypes.c_void_p(0x1008)
    def acall(**kw):
        a = dict(kn=FAKE, vn=FAKE, kc=FAKE, vc=FAKE)
        a.update(kw)
        return ap(a["kn"], a["vn"], FAKE, FAKE, FAKE, FAKE, 2, 4, 8, 8, 8, 16, 2, 64, a["kc"],
                  a["vc"], None, None)
    for key in ("kn", "vn", "kc", "vc"):
        assert acall(**{key: odd}) == INVALID, key


def test_decode_noalloc_validation(lib):
    """The no-allocation decode validates like sink_attn_decode and rejects inputs whose
    workspace would exceed its scratch array, all before any kernel launch.  A batch that
    takes whole-sequence runs writes no partials and is not rejected; it would launch, so
    here only its plan is checked (the GPU tests run it)."""
    f = lib.sink_attn_decode_noalloc
    assert lib.sink_attn_decode_noalloc_scratch_bytes() == 32 << 20
    def call(**kw):
        a = dict(q=FAKE, ind=FAKE, batch=256, ql=4, tk=256 * 32768, maxk=32768, hq=64, hkv=4,
                 d=128, ns=32, out=FAKE)
        a.update(kw)
        return f(a["q"], FAKE, FAKE, None, a["ind"], a["batch"], a["ql"], a["tk"], a["maxk"],
                 a["hq"], a["hkv"], a["d"], 0.088, 1, a["ns"], a["out"], None, None, None)
    assert call() == 6                                   # 32 forced chunks: too large
    assert lib.sink_attn_decode_plan_kind(256, 4, 64, 4, 128, 256 * 32768, 32768, 0,
                                          256) == 2      # planner: whole-sequence runs
    assert call(ns=0, tk=200 * 32768) == 6               # unequal lengths: stream partials
    assert call(q=None) == INVALID and call(out=None) == INVALID and call(ind=None) == INVALID
    assert call(ql=5) == UNSUPPORTED and call(hq=63) == INVALID and call(ns=65) == INVALID
    assert b"SCRATCH_LIMIT" in lib.sink_attn_status_str(6)


PEAK_HEADER = os.path.join(ROOT, "include", "sink_attn_peak.h")


def test_peak_library_exports_and_validates(lib):
    """The achievable-peak probes (libsinkattn_peak.so) export what include/sink_attn_peak.h
    declares and reject invalid arguments before any launch."""
    from gqa_attention_sink_amd import build as bld
    names = sorted(set(re.findall(r"^\s*int\s+(sink_attn_peak_[a-z_0-9]+)\(",
                                  open(PEAK_HEADER).read(), flags=re.M)))
    assert names == ["sink_attn_peak_coissue", "sink_attn_peak_mfma_bf16",
                     "sink_attn_peak_stream_read", "sink_attn_peak_valu"]
    out = subprocess.run(["nm", "-D", "--defined-only", bld.PEAK_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(ln.split()[-1] for ln in out.splitlines() if ln.strip())
    assert not [n for n in names if n not in exported]
    p = ctypes.CDLL(bld.PEAK_LIB)
    i32, vp = ctypes.c_int32, ctypes.c_void_p
    p.sink_attn_peak_valu.argtypes = [i32, i32, i32, i32, vp, vp]
    p.sink_attn_peak_stream_read.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
    p.sink_attn_peak_mfma_bf16.argtypes = [i32, i32, vp, vp]
    p.sink_attn_peak_coissue.argtypes = [i32, i32, i32, i32, vp, vp]
    for args in ((2, 1, 8, 1, FAKE), (0, 3, 8, 1, FAKE), (1, 1, 8, 1, None), (0, 4, 0, 1, FAKE),
                 (0, 1, 8, 0, FAKE)):
        assert p.sink_attn_peak_valu(*args, None) == 1, args
    assert p.sink_attn_peak_stream_read(FAKE, 0, 4, FAKE, None) == 1
    assert p.sink_attn_peak_stream_read(FAKE, 24, 4, FAKE, None) == 1      # not 16-byte sized
    assert p.sink_attn_peak_stream_read(ctypes.c_void_p(0x1008), 32, 4, FAKE, None) == 1
    assert p.sink_attn_peak_stream_read(FAKE, 32, 0, FAKE, None) == 1
    assert p.sink_attn_peak_mfma_bf16(0, 4, FAKE, None) == 1
    assert p.sink_attn_peak_mfma_bf16(8, 4, None, None) == 1
    assert p.sink_attn_peak_coissue(5, 0, 8, 4, FAKE, None) == 1
    assert p.sink_attn_peak_coissue(-1, 1, 8, 4, FAKE, None) == 1
