"""CPU oracle (test infrastructure only; see paged_attention.py, and fp8.py for
the 8-bit KV-cache code)."""
from .paged_attention import (  # noqa: F401
    append,
    attend,
    attend_split,
    blocks_for,
    combine,
    copy_blocks,
    gather,
    kv_cache_bytes,
    new_pool,
    paged_decode,
    paged_prefill_chunk,
    softmax_summary,
)
