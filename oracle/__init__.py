"""Independent CPU oracle for sink-aware GQA attention.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product path (``gqa_attention_sink_amd``)
never imports it, and it imports nothing from the product path.
"""
from .sink_attention import (  # noqa: F401
    sink_attention,
    sink_attention_decode,
    sink_attention_chunked,
    merge_partials,
    flops_causal,
)
from .paged_kv import (  # noqa: F401
    paged_seq_lens,
    gather_paged,
    kv_append,
    sink_attention_decode_paged,
)
from .yarn_rope import (  # noqa: F401
    yarn_inv_freq,
    yarn_mscale,
    apply_rope,
    bf16_round,
)
