"""gqa_attention_sink_amd: grouped-query attention with a learned per-head softmax sink,
as hand-written HIP kernels for MI355X (gfx950) behind a C ABI (include/sink_attn.h).

    from gqa_attention_sink_amd import prefill, decode
"""
from .sink_attn import (  # noqa: F401
    LIB_PATH,
    RopeParams,
    SinkAttnError,
    decode,
    decode_chunk_bounds,
    decode_chunks_per_slot,
    decode_noalloc,
    decode_noalloc_scratch_bytes,
    decode_num_slots,
    decode_paged,
    decode_plan_kind,
    decode_partial,
    decode_stream_merge,
    decode_stream_partial,
    decode_stream_plan,
    decode_workspace,
    decode_workspace_bytes,
    kv_append,
    load,
    merge,
    prefill,
    prefill_num_splits,
    prefill_workspace_bytes,
    rope_apply,
    version,
)
