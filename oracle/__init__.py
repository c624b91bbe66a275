"""CPU fp64 oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product (the HIP library and its Python binding) never does, and the oracle
never imports the product: the two share no code.

Every function is plain numpy in float64 and follows the vLLM pages'
definitions; see ``oracle/ref.py`` for the citation of each step.
"""

from .ref import (  # noqa: F401
    decode_bits,
    kv_bytes_per_token,
    block_bytes,
    blocks_for_tokens,
    slot_of,
    slot_mapping,
    reshape_and_cache,
    copy_blocks,
    gather_request_kv,
    paged_attention,
    paged_attention_partials,
    merge_partials,
    chunk_schedule,
    validate_metadata,
    used_slot_mask,
)
