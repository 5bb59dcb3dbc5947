"""One MLA decode step on the device: buffers plus the library calls.

Plumbing only: torch allocates the device buffers and supplies the stream;
every step of the computation runs in libmla's kernels.
"""
from __future__ import annotations

from typing import Optional

from . import _binding as B


def _torch():
    import torch
    return torch


def dtype_of(cfg: B.Config):
    t = _torch()
    return t.float32 if cfg.dtype == B.F32 else t.bfloat16


def upload(x, dtype, device="cuda"):
    """numpy -> contiguous device tensor (exact for bf16-representable values)."""
    t = _torch()
    return t.from_numpy(x).to(device=device).to(dtype).contiguous()


class DecodeStep:
    """Device state of one decode step for ``batch`` sequences of ``q_len`` tokens.

    The cache pool, page table and lengths are the caller's (shared across
    steps or rotated per layer); this object owns only the per-step buffers:
    absorbed queries, split partials, merged latent output and final output.
    """

    def __init__(self, cfg: B.Config, batch: int, q_len: int, num_splits: int,
                 seq_lens_host, device="cuda", split_chunk: int = 0, tree_parents=None,
                 cache_q8: bool = False, index_topk: int = 0, cache_bits: int = 0):
        t = _torch()
        self.cfg, self.batch, self.q_len, self.num_splits = cfg, batch, q_len, num_splits
        self.split_chunk = split_chunk  # > 0: fixed-size partitions
        # bits of the cache's codes: 0 (rows in the workload dtype), 8 or 4
        self.cache_bits = cache_bits or (8 if cache_q8 else 0)
        self.cache_q8 = self.cache_bits != 0  # (either coded format)
        H, D, dc, dv = cfg.num_heads, cfg.dim, cfg.kv_rank, cfg.v_dim
        dt = dtype_of(cfg)
        lens = [int(x) for x in seq_lens_host]
        self.max_seq_len = max(lens)
        self.tree = (None if tree_parents is None else
                     t.tensor([[int(p) for p in row] for row in tree_parents], dtype=t.int32,
                              device=device))
        # drafted token j of sequence b: cached at slot L_b - Q + j, positioned
        # there for a chain and at L_b - Q + depth(j) for a tree (derived by the
        # library from the same tree the decode masks by)
        self.seq_idx = t.empty(batch * q_len, dtype=t.int32, device=device)
        self.slot = t.empty(batch * q_len, dtype=t.int32, device=device)
        self.qpos = t.empty(batch * q_len, dtype=t.int32, device=device)
        self.set_lengths(t.tensor(lens, dtype=t.int32, device=device))
        self.q_full = t.empty((batch, q_len, H, D), dtype=dt, device=device)
        self.o_part = t.empty((batch, q_len, H, num_splits, dc), dtype=t.float32, device=device)
        self.lse_part = t.empty((batch, q_len, H, num_splits), dtype=t.float32, device=device)
        self.o_lat = t.empty((batch, q_len, H, dc), dtype=dt, device=device)
        self.lse = t.empty((batch, q_len, H), dtype=t.float32, device=device)
        self.out = t.empty((batch, q_len, H, dv), dtype=dt, device=device)
        # sparse read: index scores, then the index_topk tokens each query reads
        self.index_topk = index_topk
        if index_topk > 0:
            self.scores = t.empty((batch, q_len, self.max_seq_len), dtype=t.float32, device=device)
            self.indices = t.empty((batch, q_len, index_topk), dtype=t.int32, device=device)
            self.counts = t.empty((batch, q_len), dtype=t.int32, device=device)
            # zero once: every selection leaves it zero
            self.topk_ws = t.zeros(B.topk_workspace_bytes(batch, q_len), dtype=t.uint8,
                                   device=device)

    def set_lengths(self, seq_lens, stream=None):
        """Derive the drafted rows' slots and positions from new lengths
        (a device tensor [B] int32, each at most the max_seq_len given at
        construction)."""
        B.draft_positions(seq_lens, self.q_len, self.max_seq_len, self.tree, self.seq_idx,
                          self.slot, self.qpos, stream)

    def absorb(self, q_nope, q_rope, w_uk, stream=None):
        B.absorb_q(self.cfg, q_nope, q_rope, self.qpos, w_uk, self.q_full, stream)

    def append(self, c_new, k_new, page_table, cache, stream=None):
        if self.cache_q8:
            app = B.cache_append_q8 if self.cache_bits == 8 else B.cache_append_q4
            app(self.cfg, c_new, k_new, self.seq_idx, self.slot,
                None if self.tree is None else self.qpos, page_table, cache, B.APPEND_ROTATE,
                stream)
        elif self.tree is None:
            B.cache_append(self.cfg, c_new, k_new, self.seq_idx, self.slot, page_table, cache,
                           B.APPEND_ROTATE, stream)
        else:
            B.cache_append_at(self.cfg, c_new, k_new, self.seq_idx, self.slot, self.qpos,
                              page_table, cache, B.APPEND_ROTATE, stream)

    def index_append(self, k_idx_new, page_table, index_cache, stream=None):
        B.index_append(self.cfg, k_idx_new, self.seq_idx, self.slot, page_table, index_cache,
                       stream)

    def index_scores(self, q_idx, w_idx, index_cache, page_table, seq_lens, stream=None):
        B.index_scores(self.cfg, q_idx, w_idx, index_cache, page_table, seq_lens, self.scores,
                       self.max_seq_len, stream)

    def select(self, seq_lens, stream=None):
        B.topk_select(self.scores, seq_lens, self.indices, self.counts, self.max_seq_len,
                      self.topk_ws, stream)

    def index_select(self, q_idx, w_idx, index_cache, page_table, seq_lens, stream=None):
        """index_scores then select, as one library call."""
        B.index_scores_topk(self.cfg, q_idx, w_idx, index_cache, page_table, seq_lens,
                            self.scores, self.max_seq_len, self.indices, self.counts,
                            self.topk_ws, stream)

    def decode(self, cache, page_table, seq_lens, stream=None, max_seq_len: Optional[int] = None):
        if self.index_topk > 0:
            B.decode_sparse(self.cfg, self.q_full, cache, page_table, seq_lens, self.indices,
                            self.counts, self.o_part, self.lse_part,
                            max_seq_len or self.max_seq_len, stream)
        elif self.cache_q8:
            dec = B.decode_paged_q8 if self.cache_bits == 8 else B.decode_paged_q4
            dec(self.cfg, self.q_full, cache, page_table, seq_lens, self.o_part, self.lse_part,
                max_seq_len or self.max_seq_len, stream, chunk_tokens=self.split_chunk,
                tree_parent=self.tree)
        elif self.tree is None:
            B.decode_paged(self.cfg, self.q_full, cache, page_table, seq_lens, self.o_part,
                           self.lse_part, max_seq_len or self.max_seq_len, stream,
                           chunk_tokens=self.split_chunk)
        else:
            B.decode_paged_tree(self.cfg, self.q_full, cache, page_table, seq_lens, self.tree,
                                self.o_part, self.lse_part, max_seq_len or self.max_seq_len,
                                stream, chunk_tokens=self.split_chunk)

    def combine(self, stream=None):
        B.splitkv_combine(self.cfg, self.o_part, self.lse_part, self.o_lat, self.lse, stream)

    def up_project(self, w_uv, stream=None):
        B.up_project_v(self.cfg, self.o_lat, w_uv, self.out, stream)

    def absorb_append(self, q_nope, q_rope, w_uk, c_new, k_new, page_table, cache, stream=None):
        if self.cache_q8:
            B.absorb_append_coded(self.cfg, self.cache_bits, q_nope, q_rope, self.qpos, w_uk,
                                  self.q_full, c_new, k_new, self.seq_idx, self.slot,
                                  None if self.tree is None else self.qpos, page_table, cache,
                                  B.APPEND_ROTATE, stream)
        elif self.tree is None:
            B.absorb_append(self.cfg, q_nope, q_rope, self.qpos, w_uk, self.q_full, c_new, k_new,
                            self.seq_idx, self.slot, page_table, cache, B.APPEND_ROTATE, stream)
        else:
            B.absorb_append_at(self.cfg, q_nope, q_rope, self.qpos, w_uk, self.q_full, c_new,
                               k_new, self.seq_idx, self.slot, self.qpos, page_table, cache,
                               B.APPEND_ROTATE, stream)

    def combine_up_project(self, w_uv, stream=None):
        B.combine_up_project(self.cfg, self.o_part, self.lse_part, self.o_lat, w_uv, self.out,
                             self.lse, stream)

    def run(self, q_nope, q_rope, w_uk, w_uv, c_new, k_new, cache, page_table, seq_lens,
            stream=None, max_seq_len: Optional[int] = None, fused: bool = True, sparse=None):
        """absorb -> append (B*Q new rows) -> decode -> combine -> up-project.

        fused: the first two and the last two calls each as one library call
        (mla_absorb_append, mla_combine_up_project; same results); for a
        sparse read also the indexer-key append with the first two
        (mla_absorb_append_index) and the scoring with the selection
        (mla_index_scores_topk).
        sparse: (q_idx, w_idx, k_idx_new, index_cache) for a sparse read: the
        new indexer keys are appended, every cached token scored, the top
        index_topk selected, and the decode reads only those."""
        sparse_fused = (fused and self.index_topk > 0 and self.tree is None
                        and not self.cache_q8)
        if sparse_fused:  # absorption, latent rows and indexer keys: one call
            q_idx, w_idx, k_idx_new, index_cache = sparse
            B.absorb_append_index(self.cfg, q_nope, q_rope, self.qpos, w_uk, self.q_full, c_new,
                                  k_new, self.seq_idx, self.slot, page_table, cache, k_idx_new,
                                  index_cache, B.APPEND_ROTATE, stream)
        elif fused:
            self.absorb_append(q_nope, q_rope, w_uk, c_new, k_new, page_table, cache, stream)
        else:
            self.absorb(q_nope, q_rope, w_uk, stream)
            self.append(c_new, k_new, page_table, cache, stream)
        if self.index_topk > 0:
            q_idx, w_idx, k_idx_new, index_cache = sparse
            if not sparse_fused:
                self.index_append(k_idx_new, page_table, index_cache, stream)
            if fused:
                self.index_select(q_idx, w_idx, index_cache, page_table, seq_lens, stream)
            else:
                self.index_scores(q_idx, w_idx, index_cache, page_table, seq_lens, stream)
                self.select(seq_lens, stream)
        self.decode(cache, page_table, seq_lens, stream, max_seq_len)
        if fused:
            self.combine_up_project(w_uv, stream)
        else:
            self.combine(stream)
            self.up_project(w_uv, stream)
        return self.out


def fill_index_cache(cfg: B.Config, index_cache, page_table, k_all, seq_idx, pos, stream=None,
                     rows_per_call: int = 1 << 20):
    """Write every cached token's indexer key (setup), rows n at (seq_idx[n], pos[n])."""
    n = int(pos.numel())
    for a in range(0, n, rows_per_call):
        e = min(n, a + rows_per_call)
        B.index_append(cfg, k_all[a:e], seq_idx[a:e], pos[a:e], page_table, index_cache, stream)


def fill_cache_q8(cfg: B.Config, cache_q8, page_table, c_all, k_all, seq_idx, pos, stream=None,
                  rows_per_call: int = 1 << 20, rope_pos=None, bits: int = 8):
    """fill_cache for an 8-bit cache (cache_q8 uint8 [num_pages][page][D + 16]),
    or with bits=4 a 4-bit one ([num_pages][page][D / 2 + 16])."""
    app = B.cache_append_q8 if bits == 8 else B.cache_append_q4
    n = int(pos.numel())
    for a in range(0, n, rows_per_call):
        e = min(n, a + rows_per_call)
        app(cfg, c_all[a:e], k_all[a:e], seq_idx[a:e], pos[a:e],
            None if rope_pos is None else rope_pos[a:e], page_table, cache_q8, B.APPEND_ROTATE,
            stream)


def fill_cache(cfg: B.Config, cache, page_table, c_all, k_all, seq_idx, pos, stream=None,
               rows_per_call: int = 1 << 20, rope_pos=None):
    """Write every cached row (setup): rows n go to (seq_idx[n], pos[n]), keys
    rotated by pos[n] (rope_pos[n] when given)."""
    n = int(pos.numel())
    for a in range(0, n, rows_per_call):
        e = min(n, a + rows_per_call)
        if rope_pos is None:
            B.cache_append(cfg, c_all[a:e], k_all[a:e], seq_idx[a:e], pos[a:e], page_table, cache,
                           B.APPEND_ROTATE, stream)
        else:
            B.cache_append_at(cfg, c_all[a:e], k_all[a:e], seq_idx[a:e], pos[a:e],
                              rope_pos[a:e], page_table, cache, B.APPEND_ROTATE, stream)
