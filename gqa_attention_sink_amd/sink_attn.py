"""ctypes binding of libsinkattn.so: argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the library
is missing or no GPU is present the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SINK_ATTN_LIB may name another build of the same C ABI (the host-sanitized build that
# the CPU validation tests load); by default the in-tree HIP library.
LIB_PATH = os.environ.get("SINK_ATTN_LIB") or os.path.join(_HERE, "libsinkattn.so")

_lib = None


class RopeParams(ctypes.Structure):
    """YaRN rotary parameters (the C struct sink_attn_rope): pairs (i, i + D/2) rotate by
    pos * f_i with f_i = theta^(-2i/D), interpolated by YaRN when factor > 1."""
    _fields_ = [("theta", ctypes.c_float), ("factor", ctypes.c_float),
                ("original_max_pos", ctypes.c_int32), ("beta_fast", ctypes.c_float),
                ("beta_slow", ctypes.c_float)]

    def __init__(self, theta=10000.0, factor=1.0, original_max_pos=4096, beta_fast=32.0,
                 beta_slow=1.0):
        super().__init__(float(theta), float(factor), int(original_max_pos), float(beta_fast),
                         float(beta_slow))


_ROPE_P = ctypes.POINTER(RopeParams)

_SIGS = {  # entry points that take a rope pointer have it just before the stream
    "sink_attn_prefill": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "sink_attn_decode": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p]),
    "sink_attn_decode_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "sink_attn_decode_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "sink_attn_decode_partial": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "sink_attn_decode_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 7),
    "sink_attn_decode_num_slots": (ctypes.c_int32, [ctypes.c_int32] * 8),
    "sink_attn_decode_chunks_per_slot": (ctypes.c_int32, [ctypes.c_int32] * 8),
    "sink_attn_merge": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "sink_attn_decode_paged": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,      # q k v sinks
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,                       # page table
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64,          # b ql ent pages
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,          # ps maxkv hq hkv
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_int32,          # d scale causal ns
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "sink_attn_kv_append": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,                       # k_new v_new app
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,                       # page table
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,                          # ps hkv d
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "sink_attn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "sink_attn_last_hip_error": (ctypes.c_int, []),
    "sink_attn_version": (ctypes.c_char_p, []),
}


for _name in ("sink_attn_prefill", "sink_attn_decode", "sink_attn_decode_noalloc",
              "sink_attn_decode_partial",
              "sink_attn_decode_paged", "sink_attn_kv_append"):
    _res, _args = _SIGS[_name]
    _SIGS[_name] = (_res, _args[:-1] + [_ROPE_P, _args[-1]])
_SIGS["sink_attn_prefill_split"] = (ctypes.c_int, [
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,          # q k v sinks
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,            # cu cu b maxq
    ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,              # maxkv tq tk hq
    ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32,              # hkv d sc causal
    ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,           # ns ws wsb out
    ctypes.c_void_p, _ROPE_P, ctypes.c_void_p])
_SIGS["sink_attn_decode_stream_plan"] = (ctypes.c_int32, [
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)])
_SIGS["sink_attn_decode_plan_kind"] = (ctypes.c_int32, [
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32])
_SIGS["sink_attn_decode_chunk_bounds"] = (ctypes.c_int32, [
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32])
_SIGS["sink_attn_decode_stream_partial"] = (ctypes.c_int, [
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
    ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
    ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
    _ROPE_P, ctypes.c_void_p])
_SIGS["sink_attn_decode_stream_merge"] = (ctypes.c_int, [
    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
    ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p])
_SIGS["sink_attn_prefill_num_splits"] = (ctypes.c_int32, [ctypes.c_int32] * 7)
_SIGS["sink_attn_prefill_workspace_bytes"] = (ctypes.c_size_t, [
    ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32])
_SIGS["sink_attn_rope_apply"] = (ctypes.c_int, [
    ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
    ctypes.c_int64, ctypes.c_void_p, _ROPE_P, ctypes.c_void_p])


def _rope_arg(rope):
    if rope is None:
        return None
    _need(isinstance(rope, RopeParams), "rope must be a RopeParams")
    return ctypes.byref(rope)


def load() -> ctypes.CDLL:
    """Load (once) the in-tree HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m gqa_attention_sink_amd.build`"
                " (there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class SinkAttnError(RuntimeError):
    pass


def _check(rc: int):
    if rc != 0:
        lib = load()
        msg = lib.sink_attn_status_str(rc).decode()
        if rc == 4:
            msg += f" (hipError {lib.sink_attn_last_hip_error()})"
        raise SinkAttnError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def _dev_tensor(t: torch.Tensor, dtype, name: str, ndim: Optional[int] = None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be on the GPU")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if ndim is not None:
        _need(t.dim() == ndim, f"{name} must have {ndim} dims, got {t.dim()}")


def _sinks_arg(sinks, hq, device):
    if sinks is None:
        return None
    _dev_tensor(sinks, torch.float32, "sinks", 1)
    _need(sinks.numel() == hq and sinks.device == device, "sinks must be [Hq] on q's device")
    return sinks


def prefill(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, max_seqlen_q: int,
            sm_scale: Optional[float] = None, causal: bool = True, out=None, lse=None,
            return_lse: bool = True, rope: Optional[RopeParams] = None,
            num_splits: int = 1, max_seqlen_kv: Optional[int] = None, workspace=None):
    """Variable-length sink attention prefill.

    q [total_q, Hq, D] bf16; k, v [Hkv, total_kv, D] bf16 (HND); sinks fp32 [Hq] or
    None; cu_seqlens_q / cu_seqlens_kv int32 [B+1] on the GPU; max_seqlen_q a host int.
    num_splits != 1 splits the key axis across workgroups (0 = planner; needs
    max_seqlen_kv, a host bound of the key lengths) and merges the splits.
    Returns (out [total_q, Hq, D] bf16, lse [total_q, Hq] fp32 or None)."""
    lib = load()
    _dev_tensor(q, torch.bfloat16, "q", 3)
    _dev_tensor(k, torch.bfloat16, "k", 3)
    _dev_tensor(v, torch.bfloat16, "v", 3)
    _dev_tensor(cu_seqlens_q, torch.int32, "cu_seqlens_q", 1)
    _dev_tensor(cu_seqlens_kv, torch.int32, "cu_seqlens_kv", 1)
    tq, hq, d = q.shape
    hkv, tk, dk = k.shape
    _need(v.shape == k.shape and dk == d, "k and v must be [Hkv, total_kv, D] matching q")
    _need(cu_seqlens_q.numel() == cu_seqlens_kv.numel() and cu_seqlens_q.numel() >= 2,
          "cu_seqlens must both be [B+1]")
    batch = cu_seqlens_q.numel() - 1
    sinks = _sinks_arg(sinks, hq, q.device)
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor(out, torch.bfloat16, "out", 3)
        _need(out.shape == q.shape, "out must match q")
    if lse is None and return_lse:
        lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _dev_tensor(lse, torch.float32, "lse", 2)
        _need(tuple(lse.shape) == (tq, hq), "lse must be [total_q, Hq]")
    if num_splits == 1:
        rc = lib.sink_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q),
                                   _ptr(cu_seqlens_kv), batch, int(max_seqlen_q), tq, tk, hq,
                                   hkv, d, scale, int(bool(causal)), _ptr(out), _ptr(lse),
                                   _rope_arg(rope), _stream(q.device))
        _check(rc)
        return out, lse
    _need(max_seqlen_kv is not None, "a key-axis split needs max_seqlen_kv")
    s_res = prefill_num_splits(batch, max_seqlen_q, max_seqlen_kv, hq, hkv, num_splits)
    nbytes = prefill_workspace_bytes(tq, hq, d, s_res)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    else:
        _dev_tensor(workspace, torch.uint8, "workspace")
    rc = lib.sink_attn_prefill_split(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(cu_seqlens_q),
                                     _ptr(cu_seqlens_kv), batch, int(max_seqlen_q),
                                     int(max_seqlen_kv), tq, tk, hq, hkv, d, scale,
                                     int(bool(causal)), int(num_splits), _ptr(workspace),
                                     workspace.numel(), _ptr(out), _ptr(lse), _rope_arg(rope),
                                     _stream(q.device))
    _check(rc)
    return out, lse


def prefill_num_splits(batch: int, max_seqlen_q: int, max_seqlen_kv: int, num_q_heads: int,
                       num_kv_heads: int, num_splits: int = 0, num_cus: int = 0) -> int:
    """Resolved key-split count; num_cus = 0 plans for the current device."""
    return int(load().sink_attn_prefill_num_splits(batch, int(max_seqlen_q), int(max_seqlen_kv),
                                                   num_q_heads, num_kv_heads, int(num_splits),
                                                   int(num_cus)))


def prefill_workspace_bytes(total_q: int, num_q_heads: int, head_dim: int, splits: int) -> int:
    return int(load().sink_attn_prefill_workspace_bytes(int(total_q), num_q_heads, head_dim,
                                                        int(splits)))


def decode_chunks_per_slot(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                           head_dim: int, max_kv_len: int, num_splits: int = 0,
                           num_cus: int = 0) -> int:
    """Consecutive plan chunks whose merged state one partial slot holds."""
    return int(load().sink_attn_decode_chunks_per_slot(batch, q_len, num_q_heads, num_kv_heads,
                                                       head_dim, int(max_kv_len),
                                                       int(num_splits), int(num_cus)))


def decode_chunk_bounds(kv_len: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                        head_dim: int, num_splits: int = 0) -> list:
    """Boundaries [0, ..., kv_len] of the decode chunk plan of one sequence (chunk c
    covers keys [b[c], b[c+1]))."""
    lib = load()
    n = int(lib.sink_attn_decode_chunk_bounds(int(kv_len), q_len, num_q_heads, num_kv_heads,
                                              head_dim, int(num_splits), None, 0))
    if n == 0:
        raise SinkAttnError("invalid arguments for the decode chunk plan")
    buf = (ctypes.c_int32 * (n + 1))()
    lib.sink_attn_decode_chunk_bounds(int(kv_len), q_len, num_q_heads, num_kv_heads, head_dim,
                                      int(num_splits), buf, n + 1)
    return list(buf)


def decode_num_slots(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, max_kv_len: int, num_splits: int = 0,
                     num_cus: int = 0) -> int:
    return int(load().sink_attn_decode_num_slots(batch, q_len, num_q_heads, num_kv_heads,
                                                 head_dim, int(max_kv_len), int(num_splits),
                                                 int(num_cus)))


def decode_workspace_bytes(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                           head_dim: int, max_kv_len: int, num_splits: int = 0) -> int:
    return int(load().sink_attn_decode_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads,
                                                       head_dim, int(max_kv_len), int(num_splits)))


def decode_workspace(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, max_kv_len: int, num_splits: int = 0, device="cuda"):
    """A uint8 workspace for decode() of these sizes (contents need no initialisation);
    stream-ordered calls of any sizes it fits may share it."""
    nbytes = decode_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                    max_kv_len, num_splits)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _decode_common(q, k, v, kv_indptr):
    _dev_tensor(q, torch.bfloat16, "q", 4)
    _dev_tensor(k, torch.bfloat16, "k", 3)
    _dev_tensor(v, torch.bfloat16, "v", 3)
    _dev_tensor(kv_indptr, torch.int32, "kv_indptr", 1)
    b, ql, hq, d = q.shape
    hkv, tk, dk = k.shape
    _need(v.shape == k.shape and dk == d, "k and v must be [Hkv, total_kv, D] matching q")
    _need(kv_indptr.numel() == b + 1, "kv_indptr must be [batch+1]")
    return b, ql, hq, d, hkv, tk


def decode(q, k, v, sinks, kv_indptr, max_kv_len: int, sm_scale: Optional[float] = None,
           causal: bool = True, num_splits: int = 0, workspace=None, out=None, lse=None,
           return_lse: bool = True, rope: Optional[RopeParams] = None):
    """Split-KV decode with log-sum-exp merge.

    q [B, q_len, Hq, D] bf16 (q_len 1..4); k, v [Hkv, total_kv, D] bf16 (HND);
    kv_indptr int32 [B+1] (the KV already holds the q_len new tokens); max_kv_len a
    host int.  workspace: a uint8 GPU tensor of at least decode_workspace_bytes(...)
    bytes (decode_workspace() makes one; allocated here if None).  Returns (out [B, q_len, Hq, D], lse [B, q_len, Hq])."""
    lib = load()
    b, ql, hq, d, hkv, tk = _decode_common(q, k, v, kv_indptr)
    sinks = _sinks_arg(sinks, hq, q.device)
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    nbytes = decode_workspace_bytes(b, ql, hq, hkv, d, max_kv_len, num_splits)
    if workspace is None:
        workspace = decode_workspace(b, ql, hq, hkv, d, max_kv_len, num_splits, q.device)
    else:
        _dev_tensor(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev_tensor(out, torch.bfloat16, "out", 4)
        _need(out.shape == q.shape, "out must match q")
    if lse is None and return_lse:
        lse = torch.empty((b, ql, hq), dtype=torch.float32, device=q.device)
    rc = lib.sink_attn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(kv_indptr), b, ql,
                              tk, int(max_kv_len), hq, hkv, d, scale, int(bool(causal)),
                              int(num_splits), _ptr(workspace), workspace.numel(), _ptr(out),
                              _ptr(lse), _rope_arg(rope), _stream(q.device))
    _check(rc)
    return out, lse


def decode_noalloc(q, k, v, sinks, kv_indptr, max_kv_len: int, out, lse=None,
                   sm_scale: Optional[float] = None, causal: bool = True, num_splits: int = 0,
                   rope: Optional[RopeParams] = None):
    """decode() through the entry point that allocates nothing: the partials live in the
    library's per-GPU scratch array (decode_noalloc_scratch_bytes() bytes), so `out`
    (and `lse`, if wanted) must be given.  Calls that may overlap on one GPU race."""
    lib = load()
    b, ql, hq, d, hkv, tk = _decode_common(q, k, v, kv_indptr)
    sinks = _sinks_arg(sinks, hq, q.device)
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    _dev_tensor(out, torch.bfloat16, "out", 4)
    _need(out.shape == q.shape, "out must match q")
    if lse is not None:
        _dev_tensor(lse, torch.float32, "lse", 3)
        _need(tuple(lse.shape) == (b, ql, hq), "lse must be [B, q_len, Hq]")
    rc = lib.sink_attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(kv_indptr),
                                      b, ql, tk, int(max_kv_len), hq, hkv, d, scale,
                                      int(bool(causal)), int(num_splits), _ptr(out), _ptr(lse),
                                      _rope_arg(rope), _stream(q.device))
    _check(rc)
    return out, lse


def decode_noalloc_scratch_bytes() -> int:
    return int(load().sink_attn_decode_noalloc_scratch_bytes())


def decode_partial(q, k, v, sinks, kv_indptr, max_kv_len: int, sm_scale: Optional[float] = None,
                   causal: bool = True, num_splits: int = 0, part_o=None, part_lse=None,
                   rope: Optional[RopeParams] = None):
    """First stage of decode alone.  Returns (part_o [B*q_len*Hq, S, D] fp32,
    part_lse [B*q_len*Hq, S] fp32) with S = decode_num_slots(B, q_len, Hq, Hkv, D,
    max_kv_len, num_splits); slot j holds plan chunks [j*C, j*C + C), C =
    decode_chunks_per_slot(...)."""
    lib = load()
    b, ql, hq, d, hkv, tk = _decode_common(q, k, v, kv_indptr)
    sinks = _sinks_arg(sinks, hq, q.device)
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    s = decode_num_slots(b, ql, hq, hkv, d, max_kv_len, num_splits)
    rows = b * ql * hq
    if part_o is None:
        part_o = torch.empty((rows, s, d), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((rows, s), dtype=torch.float32, device=q.device)
    _dev_tensor(part_o, torch.float32, "part_o", 3)
    _dev_tensor(part_lse, torch.float32, "part_lse", 2)
    _need(tuple(part_o.shape) == (rows, s, d) and tuple(part_lse.shape) == (rows, s),
          "partial buffers have the wrong shape")
    rc = lib.sink_attn_decode_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(kv_indptr),
                                      b, ql, tk, int(max_kv_len), hq, hkv, d, scale,
                                      int(bool(causal)), int(num_splits), _ptr(part_o),
                                      _ptr(part_lse), _rope_arg(rope), _stream(q.device))
    _check(rc)
    return part_o, part_lse


DECODE_PLANS = {0: "chunks", 1: "stream", 2: "whole_runs"}


def decode_plan_kind(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                     head_dim: int, total_kv: int, max_kv_len: int, num_splits: int = 0,
                     num_cus: int = 0) -> str:
    """Which plan decode() uses for these sizes (contiguous K/V): "chunks", "stream" or
    "whole_runs".  num_cus = 0 plans for the current device."""
    k = load().sink_attn_decode_plan_kind(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                          int(total_kv), int(max_kv_len), int(num_splits),
                                          int(num_cus))
    if k < 0:
        raise ValueError("invalid decode sizes")
    return DECODE_PLANS[k]


def decode_stream_plan(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int,
                       head_dim: int, total_kv: int, max_kv_len: int, num_cus: int = 0):
    """(R, ranges_per_head, slots) of the stream plan for these sizes (what the stream
    step entry points use, and decode() too unless decode_plan_kind() says
    "whole_runs"), or None when it does not apply.  num_cus = 0 plans for the current
    device."""
    r, n, s = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    ok = load().sink_attn_decode_stream_plan(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                             int(total_kv), int(max_kv_len), int(num_cus),
                                             ctypes.byref(r), ctypes.byref(n), ctypes.byref(s))
    return (r.value, n.value, s.value) if ok else None


def _stream_views(workspace, rows: int, slots: int, d: int):
    ob = (rows * slots * d * 4 + 255) // 256 * 256
    po = workspace[: rows * slots * d * 4].view(torch.float32).view(rows, slots, d)
    pl = workspace[ob: ob + rows * slots * 4].view(torch.float32).view(rows, slots)
    return po, pl


def decode_stream_partial(q, k, v, kv_indptr, max_kv_len: int, sm_scale: Optional[float] = None,
                          causal: bool = True, workspace=None, rope: Optional[RopeParams] = None):
    """First step of the stream plan alone.  Returns (part_o [rows, S, D] fp32, part_lse
    [rows, S] fp32, workspace): views into the workspace; slot j of a row holds the keys of
    its sequence in range floor(kv_indptr[b]/R) + j (no sink); slots past the sequence's
    last range are not written."""
    lib = load()
    b, ql, hq, d, hkv, tk = _decode_common(q, k, v, kv_indptr)
    plan = decode_stream_plan(b, ql, hq, hkv, d, tk, max_kv_len)
    _need(plan is not None, "the stream plan does not apply to these sizes")
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    if workspace is None:
        workspace = decode_workspace(b, ql, hq, hkv, d, max_kv_len, 0, q.device)
    _dev_tensor(workspace, torch.uint8, "workspace")
    rc = lib.sink_attn_decode_stream_partial(_ptr(q), _ptr(k), _ptr(v), _ptr(kv_indptr), b, ql,
                                             tk, int(max_kv_len), hq, hkv, d, scale,
                                             int(bool(causal)), _ptr(workspace),
                                             workspace.numel(), _rope_arg(rope),
                                             _stream(q.device))
    _check(rc)
    po, pl = _stream_views(workspace, b * ql * hq, plan[2], d)
    return po, pl, workspace


def decode_stream_merge(sinks, kv_indptr, q_shape, total_kv: int, num_kv_heads: int,
                        max_kv_len: int, workspace, out=None, lse=None):
    """Second step of the stream plan alone: (out [B, q_len, Hq, D] bf16, lse [B, q_len, Hq])
    from the partials in `workspace` and the sinks."""
    lib = load()
    b, ql, hq, d = q_shape
    _dev_tensor(kv_indptr, torch.int32, "kv_indptr", 1)
    _dev_tensor(workspace, torch.uint8, "workspace")
    sinks = _sinks_arg(sinks, hq, workspace.device)
    if out is None:
        out = torch.empty((b, ql, hq, d), dtype=torch.bfloat16, device=workspace.device)
    if lse is None:
        lse = torch.empty((b, ql, hq), dtype=torch.float32, device=workspace.device)
    rc = lib.sink_attn_decode_stream_merge(_ptr(sinks), _ptr(kv_indptr), b, ql, int(total_kv),
                                           int(max_kv_len), hq, num_kv_heads, d, _ptr(workspace),
                                           workspace.numel(), _ptr(out), _ptr(lse),
                                           _stream(workspace.device))
    _check(rc)
    return out, lse


def merge(part_o, part_lse, out=None, lse=None, return_lse: bool = True, splits_per_row=None):
    """Log-sum-exp merge of partials: part_o [rows, S, D] fp32, part_lse [rows, S] fp32
    -> (out [rows, D] bf16, lse [rows] fp32).  splits_per_row: optional int32 [rows], the
    number of leading slots each row merges (None = all S)."""
    lib = load()
    _dev_tensor(part_o, torch.float32, "part_o", 3)
    _dev_tensor(part_lse, torch.float32, "part_lse", 2)
    rows, s, d = part_o.shape
    _need(tuple(part_lse.shape) == (rows, s), "part_lse must be [rows, S]")
    if splits_per_row is not None:
        _dev_tensor(splits_per_row, torch.int32, "splits_per_row", 1)
        _need(splits_per_row.numel() == rows, "splits_per_row must be [rows]")
    if out is None:
        out = torch.empty((rows, d), dtype=torch.bfloat16, device=part_o.device)
    if lse is None and return_lse:
        lse = torch.empty((rows,), dtype=torch.float32, device=part_o.device)
    rc = lib.sink_attn_merge(_ptr(part_o), _ptr(part_lse), _ptr(splits_per_row), rows, s, d,
                             _ptr(out), _ptr(lse), _stream(part_o.device))
    _check(rc)
    return out, lse


def version() -> str:
    return load().sink_attn_version().decode()


def _page_table(kv_page_indptr, kv_page_indices, kv_last_page_len, batch):
    _dev_tensor(kv_page_indptr, torch.int32, "kv_page_indptr", 1)
    _dev_tensor(kv_page_indices, torch.int32, "kv_page_indices", 1)
    _dev_tensor(kv_last_page_len, torch.int32, "kv_last_page_len", 1)
    _need(kv_page_indptr.numel() == batch + 1, "kv_page_indptr must be [batch+1]")
    _need(kv_last_page_len.numel() == batch, "kv_last_page_len must be [batch]")


def _cache_dims(k_cache, v_cache):
    _dev_tensor(k_cache, torch.bfloat16, "k_cache", 4)
    _dev_tensor(v_cache, torch.bfloat16, "v_cache", 4)
    _need(k_cache.shape == v_cache.shape, "k_cache and v_cache must match")
    return k_cache.shape  # num_pages, Hkv, page_size, D


def decode_paged(q, k_cache, v_cache, sinks, kv_page_indptr, kv_page_indices,
                 kv_last_page_len, max_kv_len: int, sm_scale: Optional[float] = None,
                 causal: bool = True, num_splits: int = 0, workspace=None, out=None, lse=None,
                 return_lse: bool = True, rope: Optional[RopeParams] = None):
    """Decode over a paged cache [num_pages, Hkv, page_size, D] (HND inside a page).
    q [B, q_len, Hq, D] bf16.  Returns (out [B, q_len, Hq, D], lse [B, q_len, Hq])."""
    lib = load()
    _dev_tensor(q, torch.bfloat16, "q", 4)
    b, ql, hq, d = q.shape
    num_pages, hkv, ps, dk = _cache_dims(k_cache, v_cache)
    _need(dk == d, "cache head_dim must match q")
    _page_table(kv_page_indptr, kv_page_indices, kv_last_page_len, b)
    sinks = _sinks_arg(sinks, hq, q.device)
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    if workspace is None:
        workspace = decode_workspace(b, ql, hq, hkv, d, max_kv_len, num_splits, q.device)
    else:
        _dev_tensor(workspace, torch.uint8, "workspace")
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((b, ql, hq), dtype=torch.float32, device=q.device)
    rc = lib.sink_attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(sinks),
                                    _ptr(kv_page_indptr), _ptr(kv_page_indices),
                                    _ptr(kv_last_page_len), b, ql, kv_page_indices.numel(),
                                    num_pages, ps, int(max_kv_len), hq, hkv, d, scale,
                                    int(bool(causal)), int(num_splits), _ptr(workspace),
                                    workspace.numel(), _ptr(out), _ptr(lse), _rope_arg(rope),
                                    _stream(q.device))
    _check(rc)
    return out, lse


def kv_append(k_new, v_new, append_indptr, kv_page_indptr, kv_page_indices, kv_last_page_len,
              k_cache, v_cache, max_append_len: int, rope: Optional[RopeParams] = None):
    """Write k_new/v_new [total_new, Hkv, D] into the paged caches in place (the page table
    already counts the new tokens)."""
    lib = load()
    _dev_tensor(k_new, torch.bfloat16, "k_new", 3)
    _dev_tensor(v_new, torch.bfloat16, "v_new", 3)
    _need(k_new.shape == v_new.shape, "k_new and v_new must match")
    _dev_tensor(append_indptr, torch.int32, "append_indptr", 1)
    b = append_indptr.numel() - 1
    num_pages, hkv, ps, d = _cache_dims(k_cache, v_cache)
    _need(k_new.shape[1] == hkv and k_new.shape[2] == d, "k_new must be [total_new, Hkv, D]")
    _page_table(kv_page_indptr, kv_page_indices, kv_last_page_len, b)
    rc = lib.sink_attn_kv_append(_ptr(k_new), _ptr(v_new), _ptr(append_indptr),
                                 _ptr(kv_page_indptr), _ptr(kv_page_indices),
                                 _ptr(kv_last_page_len), b, int(max_append_len),
                                 k_new.shape[0], kv_page_indices.numel(), num_pages, ps, hkv, d,
                                 _ptr(k_cache), _ptr(v_cache), _rope_arg(rope),
                                 _stream(k_new.device))
    _check(rc)
    return k_cache, v_cache


def rope_apply(x, positions, rope: RopeParams, token_dim: int = 0, head_dim_axis: int = 1):
    """Rotate a bf16 tensor in place: x has a token axis, a head axis and a last axis of
    size D (e.g. [total, H, D] with token_dim=0, head_dim_axis=1, or HND keys
    [Hkv, total, D] with token_dim=1, head_dim_axis=0); token t at positions[t]."""
    lib = load()
    _need(isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 3,
          "x must be a 3-d bf16 GPU tensor")
    _need(x.stride(-1) == 1, "the last axis of x must be contiguous")
    _dev_tensor(positions, torch.int32, "positions", 1)
    tokens, heads, d = x.shape[token_dim], x.shape[head_dim_axis], x.shape[-1]
    _need(positions.numel() == tokens, "positions must have one entry per token")
    rc = lib.sink_attn_rope_apply(_ptr(x), tokens, heads, d, x.stride(token_dim),
                                  x.stride(head_dim_axis), _ptr(positions), _rope_arg(rope),
                                  _stream(x.device))
    _check(rc)
    return x
