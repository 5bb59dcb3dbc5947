"""MLA latent-cache decode on MI355X (gfx950): Python binding of libmla.so.

The binding only marshals arguments: it checks tensor dtypes, devices and
sizes on the host (the C ABI sees raw pointers and cannot), then calls the
entry point of the same name in libmla.so on the current torch stream. Every
step of the decode path runs in the library's HIP kernels; there is no
fallback. If the library is missing, every call raises.

    cfg = Config(num_heads=16, kv_rank=512, rope_dim=64, nope_dim=128, v_dim=128)
    absorb_q(cfg, q_nope, q_rope, pos, w_uk, q_full)
    cache_append(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache)
    decode_paged(cfg, q_full, cache, page_table, seq_lens, o_part, lse_part, max_seq_len)
    splitkv_combine(cfg, o_part, lse_part, o_lat, lse)
    up_project_v(cfg, o_lat, w_uv, out)

absorb_append and combine_up_project run the first two and the last two of
these calls in one launch each, with the same results. A tree of drafted
tokens is verified with draft_positions (each drafted row's slot and RoPE
position, derived on the device from the tree), cache_append_at /
absorb_append_at and decode_paged_tree. An 8-bit latent cache (uint8 rows
of codes plus per-part min and step) is written by cache_append_q8 and read
by decode_paged_q8; a 4-bit one (two codes per byte) by cache_append_q4 and
decode_paged_q4 (absorb_append_coded runs the absorption and either coded
append in one launch). A sparse read (attention over the top-scored tokens
only) runs index_append, index_scores, topk_select and decode_sparse.
"""
from ._binding import (  # noqa: F401
    F32,
    BF16,
    APPEND_RAW,
    APPEND_ROTATE,
    Config,
    MLAError,
    lib,
    lib_path,
    build_info,
    status_str,
    config_validate,
    cache_bytes_per_token,
    split_chunk,
    default_num_splits,
    decode_partials_bytes,
    decode_kernel_kind,
    absorb_q,
    cache_append,
    decode_paged,
    splitkv_combine,
    up_project_v,
    absorb_append,
    combine_up_project,
    chunk_plan,
    cache_append_at,
    absorb_append_at,
    decode_paged_tree,
    cache_q8_bytes_per_token,
    cache_append_q8,
    decode_paged_q8,
    cache_q4_bytes_per_token,
    cache_append_q4,
    decode_paged_q4,
    index_append,
    index_scores,
    index_scores_topk,
    topk_select,
    topk_workspace_bytes,
    sparse_chunk,
    decode_sparse_kernel_kind,
    decode_sparse,
    draft_positions,
    stream_read,
    index_scores_topk_noalloc,
    TOPK_NOALLOC_MAX_QUERIES,
    prefill_workspace_bytes,
    prefill_form,
    prefill_unabsorbed,
    absorb_append_coded,
    absorb_append_index,
)
