"""fp64 CPU oracle for MLA latent-cache decode (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the HIP library and its binding never do.
"""
from . import mla_ref, brute  # noqa: F401
from .mla_ref import (  # noqa: F401
    latent_bytes_per_token,
    per_head_kv_bytes_per_token,
    rope_freqs,
    rope,
    expand_kv,
    query_positions,
    tree_depths,
    tree_ancestry,
    tree_positions,
    tree_excluded,
    attend_scores,
    attend_sequence,
    mla_decode_ref,
    absorbed_query,
    absorbed_attend_sequence,
    split_bounds,
    attend_partials,
    lse_combine,
    cache_slot,
    cache_append_image,
    Q8_LEVELS,
    quantize_q8,
    dequantize_q8,
    quantize_cache_rows,
    rotated_keys_f32,
    attend_sequence_rotated,
    mla_decode_ref_q8,
    Q4_LEVELS,
    quantize_q4,
    pack_q4,
    unpack_q4,
    mla_decode_ref_q4,
    indexer_scores,
    topk_tokens,
    dsa_selection,
    mla_decode_ref_sparse,
    prefill_in_chunks,
)
from .brute import brute_sequence, brute_index_scores  # noqa: F401
