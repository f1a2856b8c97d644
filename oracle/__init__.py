"""Plain fp64 CPU oracle for paged-KV-cache attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``paged_kv_cache_pa_amd``) never imports it and shares no code with it.
"""

from .pa_oracle import (  # noqa: F401
    attention,
    attention_buggy_clamp,
    attention_loops,
    attention_partial,
    combine_partials,
    flex_attention_dense,
    gather_sequence,
    scatter_kv,
    sdpa,
    seq_of_token,
    slots_from_block_table,
    softcap_scores,
    validate_metadata,
)
