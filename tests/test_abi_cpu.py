"""C ABI of libmla on the CPU: the library loads, exports every declared entry
point, and its host-side checks and sizing behave as documented. No call here
reaches a kernel launch (every call either fails validation or is a no-op)."""
import ctypes
import os
import re

import pytest

import oracle
import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

mla = pytest.importorskip("mla_latent_kv_03_amd")


@pytest.fixture(scope="module")
def L():
    try:
        return mla.lib()
    except RuntimeError as e:
        pytest.fail(f"libmla.so must be built before the tests: {e}")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ["mla_absorb_q", "mla_cache_append", "mla_decode_paged", "mla_splitkv_combine",
              "mla_up_project_v"]:
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name
    assert "gfx950" in mla.build_info()


V2 = mla.Config(num_heads=16)
TINY = mla.Config(num_heads=4, kv_rank=64, rope_dim=16, nope_dim=32, v_dim=32, dtype=mla.F32)


def test_config_validation_codes(L):
    assert mla.config_validate(V2) == 0
    assert mla.config_validate(TINY) == 0
    bad = {
        2: [V2.__class__(num_heads=0), V2.__class__(num_heads=16, rope_dim=3),
            V2.__class__(num_heads=16, page_size=48), V2.__class__(num_heads=16, kv_rank=500),
            V2.__class__(num_heads=16, softmax_scale=-1.0)],
        3: [V2.__class__(num_heads=16, dtype=7)],
    }
    for code, cfgs in bad.items():
        for c in cfgs:
            assert mla.config_validate(c) == code, c
    assert L.mla_config_validate(None) == 1


def test_status_strings(L):
    for s in range(8):
        assert mla.status_str(s).startswith("MLA_")
    assert "unknown" in mla.status_str(99)


def test_cache_bytes_per_token_matches_pages(L):
    assert mla.cache_bytes_per_token(V2) == 1152
    assert mla.cache_bytes_per_token(V2) * 27 == oracle.latent_bytes_per_token(512, 64, 2, 27) == 31104
    assert mla.cache_bytes_per_token(TINY) == 320
    assert mla.cache_bytes_per_token(V2.__class__(num_heads=0)) == 0


@pytest.mark.parametrize("page", [16, 64, 128])
def test_split_plan_matches_oracle(L, page):
    cfg = mla.Config(num_heads=16, page_size=page)
    for Lq in [1, 15, 16, 63, 64, 65, 1000, 32768, 1048576]:
        for S in [1, 3, 7, 32, 256, 4096]:
            chunk = mla.split_chunk(cfg, Lq, S)
            want = oracle.split_bounds(Lq, S, page)
            got = [(min(Lq, s * chunk), min(Lq, (s + 1) * chunk)) for s in range(S)]
            assert got == want, (Lq, S)


def test_chunk_plan(L):
    cfg = mla.Config(num_heads=16)
    # V2-Lite varlen batch: ~568K tokens over 256 CUs -> about 6 partitions per CU
    ck, ns = mla.chunk_plan(cfg, 568107, 32768, 256)
    assert ck % 64 == 0 and ck * ns >= 32768 and (ns - 1) * ck < 32768
    assert 4 * 256 <= 568107 / ck <= 8 * 256
    ck, ns = mla.chunk_plan(cfg, 100, 100, 256)          # tiny batch: one page
    assert (ck, ns) == (64, 2)
    ck, ns = mla.chunk_plan(cfg, 1 << 30, 1 << 30, 256)  # at most 4096 partitions
    assert ns <= 4096 and ck * ns >= 1 << 30
    with pytest.raises(mla.MLAError):
        mla.chunk_plan(cfg, 0, 10, 256)


def test_partials_bytes_and_default_splits(L):
    assert mla.decode_partials_bytes(V2, 8, 1, 32) == 8 * 16 * 32 * 513 * 4
    assert mla.decode_partials_bytes(V2, 8, 1, 0) == 0
    for wl in workload.WORKLOADS.values():
        cfg = mla.Config.from_workload(wl)
        s = mla.default_num_splits(cfg, wl.batch, wl.q_len, wl.max_seq_len, 256)
        assert 1 <= s <= 4096


def test_decode_kernel_selection(L):
    assert mla.decode_kernel_kind(V2, 1) == "mfma_rows16"
    assert mla.decode_kernel_kind(mla.Config(num_heads=128), 4) == "mfma_ws"
    assert mla.decode_kernel_kind(mla.Config(num_heads=128, page_size=16), 1) == "mfma_ws"
    assert mla.decode_kernel_kind(mla.Config(num_heads=48), 1) == "mfma_rows16"  # 48 rows
    assert mla.decode_kernel_kind(TINY, 1) == "generic"
    assert mla.decode_kernel_kind(mla.Config(num_heads=4), 1) == "generic"  # 4 rows < 16


P = ctypes.c_void_p
A16 = P(0x10000)      # aligned, never dereferenced: every call below fails first
MIS = P(0x10008)


def _c(cfg):
    return ctypes.byref(cfg.c())


def test_absorb_errors(L):
    assert L.mla_absorb_q(_c(V2), 4, None, A16, A16, A16, A16, None) == 1
    assert L.mla_absorb_q(_c(V2), 4, MIS, A16, A16, A16, A16, None) == 4
    assert L.mla_absorb_q(_c(V2), -1, A16, A16, A16, A16, A16, None) == 2
    assert L.mla_absorb_q(_c(V2), 0, None, None, None, None, None, None) == 0   # no-op
    assert L.mla_absorb_q(None, 4, A16, A16, A16, A16, A16, None) == 1


def test_append_errors(L):
    args = [A16, A16, A16, A16, A16]
    assert L.mla_cache_append(_c(V2), 8, *args, 2, 4, None, 16, 1, None) == 1
    assert L.mla_cache_append(_c(V2), 8, *args, 2, 4, A16, 16, 5, None) == 2     # bad mode
    assert L.mla_cache_append(_c(V2), 8, *args, 0, 4, A16, 16, 1, None) == 2     # batch 0
    assert L.mla_cache_append(_c(V2), 8, MIS, *args[1:], 2, 4, A16, 16, 1, None) == 4
    assert L.mla_cache_append(_c(V2), 0, *args, 2, 4, A16, 16, 1, None) == 0     # no-op


def test_decode_errors(L):
    def call(cfg=V2, batch=2, q_len=1, S=4, max_seq=256, npages=8, max_pages=4, o=A16, q=A16):
        return L.mla_decode_paged(_c(cfg), batch, q_len, S, max_seq, q, A16, npages, A16,
                                  max_pages, A16, o, A16, None)
    assert call(o=None) == 1
    assert call(q=MIS) == 4
    assert call(S=0) == 2 and call(S=4097) == 2
    assert call(max_seq=257) == 5            # 4 pages x 64 < 257
    assert call(q_len=5, max_seq=4) == 5     # q_len > max_seq_len
    assert call(q_len=0) == 2
    assert call(cfg=V2.__class__(num_heads=16, dtype=9)) == 3
    assert call(batch=0) == 0                # nothing to do


def test_combine_and_up_errors(L):
    assert L.mla_splitkv_combine(_c(V2), 2, 1, 4, None, A16, A16, None, None) == 1
    assert L.mla_splitkv_combine(_c(V2), 2, 1, 4, A16, A16, A16, MIS, None) == 4
    assert L.mla_splitkv_combine(_c(V2), 2, 1, 0, A16, A16, A16, None, None) == 2
    assert L.mla_up_project_v(_c(V2), 3, A16, None, A16, None) == 1
    assert L.mla_up_project_v(_c(V2), 0, None, None, None, None) == 0


def test_chunked_decode_errors(L):
    def call(chunk=64, S=4, max_seq=256, batch=2, o=A16):
        return L.mla_decode_paged_chunked(_c(V2), batch, 1, chunk, S, max_seq, A16, A16, 8, A16,
                                          4, A16, o, A16, None)
    assert call(chunk=0) == 2 and call(chunk=100) == 2      # not a positive multiple of the page
    assert call(chunk=64, S=2) == 5                          # 2 x 64 tokens < max_seq_len 256
    assert call(S=0) == 2
    assert call(o=None) == 1
    assert call(batch=0) == 0


def test_fused_call_errors(L):
    a = [A16] * 5
    # absorb arguments are checked first, then the append arguments
    assert L.mla_absorb_append(_c(V2), 4, None, *a[:4], 4, *a, 2, 4, A16, 16, 1, None) == 1
    assert L.mla_absorb_append(_c(V2), 4, *a, 4, *a, 2, 4, None, 16, 1, None) == 1
    assert L.mla_absorb_append(_c(V2), 4, *a, 4, *a, 2, 4, A16, 16, 7, None) == 2
    assert L.mla_absorb_append(_c(V2), 0, *[None] * 5, 0, *[None] * 5, 1, 1, None, 1, 1,
                               None) == 0
    assert L.mla_combine_up_project(_c(V2), 2, 1, 4, A16, A16, A16, None, None, A16, None) == 1
    assert L.mla_combine_up_project(_c(V2), 2, 1, 4, A16, A16, A16, MIS, A16, A16, None) == 4
    assert L.mla_combine_up_project(_c(V2), 0, 1, 4, None, None, None, None, None, None,
                                    None) == 0


def test_tree_decode_errors(L):
    def call(q_len=8, chunk=0, S=4, max_seq=256, batch=2, tree=A16, o=A16):
        return L.mla_decode_paged_tree(_c(V2), batch, q_len, chunk, S, max_seq, A16, A16, 8, A16,
                                       4, A16, tree, o, A16, None)
    assert call(tree=None) == 1
    assert call(tree=MIS) == 4
    assert call(q_len=65) == 2 and call(q_len=0) == 2        # one 64-bit branch mask per query
    assert call(chunk=100) == 2 and call(chunk=64, S=2) == 5  # as the fixed-size plan
    assert call(S=0) == 2
    assert call(o=None) == 1
    assert call(batch=0, tree=None) == 0                     # nothing to do


def test_append_at_errors(L):
    args = [A16, A16, A16, A16]
    # c_kv, k_rope, seq_idx, pos, rope_pos, page_table, batch, max_pages, cache, num_pages, flags
    assert L.mla_cache_append_at(_c(V2), 8, *args, MIS, A16, 2, 4, A16, 16, 1, None) == 4
    assert L.mla_cache_append_at(_c(V2), 8, *args, A16, None, 2, 4, A16, 16, 1, None) == 1
    assert L.mla_cache_append_at(_c(V2), 8, *args, A16, A16, 2, 4, A16, 16, 3, None) == 2
    assert L.mla_cache_append_at(_c(V2), 0, *args, None, A16, 2, 4, A16, 16, 1, None) == 0
    a = [A16] * 5
    assert L.mla_absorb_append_at(_c(V2), 4, *a, 4, *args, MIS, A16, 2, 4, A16, 16, 1,
                                  None) == 4
    assert L.mla_absorb_append_at(_c(V2), 4, None, *a[:4], 4, *args, A16, A16, 2, 4, A16, 16, 1,
                                  None) == 1


def test_draft_positions_errors(L):
    # batch, q_len, max_seq_len, seq_lens, tree_parent, seq_idx, slot, pos, stream
    def call(batch=2, q_len=4, max_len=64, lens=A16, tree=A16, si=A16, sl=A16, pos=A16):
        return L.mla_draft_positions(batch, q_len, max_len, lens, tree, si, sl, pos, None)
    assert call(q_len=0) == 2 and call(batch=-1) == 2
    assert call(q_len=65) == 2                                 # one 64-bit branch mask per query
    assert call(q_len=65, tree=None, max_len=64) == 5          # q_len above max_seq_len
    assert call(lens=None) == 1 and call(pos=None) == 1 and call(si=MIS) == 4
    assert call(tree=MIS) == 4
    assert call(batch=0, lens=None) == 0                       # nothing to do


def test_stream_read_errors(L):
    assert L.mla_stream_read(A16, 24, A16, 4, None) == 2       # not a multiple of 16
    assert L.mla_stream_read(A16, 32, A16, 0, None) == 2
    assert L.mla_stream_read(None, 32, A16, 4, None) == 1
    assert L.mla_stream_read(MIS, 32, A16, 4, None) == 4
    assert L.mla_stream_read(None, 0, None, 4, None) == 0      # nothing to read


def test_q8_entry_errors(L):
    assert L.mla_cache_q8_bytes_per_token(_c(V2)) == 592
    assert L.mla_cache_q8_bytes_per_token(_c(TINY)) == 96          # 64 + 16 codes + 16
    def dec(cfg=V2, q_len=1, batch=2, chunk=0, S=4, tree=None, o=A16, max_pages=4):
        return L.mla_decode_paged_q8(_c(cfg), batch, q_len, chunk, S, 256, A16, A16, 8, A16,
                                     max_pages, A16, tree, o, A16, None)
    assert dec(o=None) == 1
    assert dec(tree=MIS) == 4
    assert dec(q_len=65, tree=A16) == 2                              # tree mask limit
    assert dec(cfg=mla.Config(num_heads=16, page_size=32), max_pages=8) == 6  # tile > page
    assert dec(cfg=mla.Config(num_heads=8)) == 6                     # 8 rows: no kernel
    assert dec(cfg=TINY) == 6                                        # fp32 / other shapes
    assert dec(batch=0) == 0
    args = [A16, A16, A16, A16]
    assert L.mla_cache_append_q8(_c(V2), 8, *args, MIS, A16, 2, 4, A16, 16, 1, None) == 4
    assert L.mla_cache_append_q8(_c(V2), 8, *args, None, A16, 2, 4, None, 16, 1, None) == 1
    odd = mla.Config(num_heads=4, kv_rank=64, rope_dim=8, nope_dim=32, v_dim=32, dtype=mla.F32)
    assert L.mla_cache_append_q8(_c(odd), 8, *args, None, A16, 2, 4, A16, 16, 1, None) == 6


def test_absorb_append_index_errors(L):
    a5 = [A16] * 5
    f = L.mla_absorb_append_index
    def call(q=A16, k_idx=A16, icache=A16, dI=128, flags=1, n_app=4, cache=A16):
        return f(_c(V2), 4, q, *a5[1:], n_app, A16, A16, A16, A16, A16, 2, 4, cache, 16, flags, dI,
                 k_idx, icache, None)
    assert call(q=None) == 1                   # absorb arguments first
    assert call(cache=None) == 1               # then the append's
    assert call(flags=7) == 2
    assert call(dI=100) == 2                   # then the indexer's: a multiple of 8
    assert call(dI=0) == 2
    assert call(k_idx=None) == 1
    assert call(icache=MIS) == 4
    assert f(_c(V2), 0, *[None] * 5, 0, *[None] * 5, 1, 1, None, 1, 1, 128, None, None, None) == 0


def test_coded_absorb_append_errors(L):
    a5 = [A16] * 5
    for name in ("mla_absorb_append_q8", "mla_absorb_append_q4"):
        f = getattr(L, name)
        # absorb arguments first, then the append's, then the coded row shape
        assert f(_c(V2), 4, None, *a5[:4], 4, A16, A16, A16, A16, None, A16, 2, 4, A16, 16, 1,
                 None) == 1
        assert f(_c(V2), 4, *a5, 4, A16, A16, A16, A16, None, A16, 2, 4, None, 16, 1, None) == 1
        assert f(_c(V2), 4, *a5, 4, A16, A16, A16, A16, MIS, A16, 2, 4, A16, 16, 1, None) == 4
        assert f(_c(V2), 4, *a5, 4, A16, A16, A16, A16, None, A16, 2, 4, A16, 16, 7, None) == 2
        odd = mla.Config(num_heads=4, kv_rank=64, rope_dim=8, nope_dim=32, v_dim=32,
                         dtype=mla.F32)
        assert f(_c(odd), 4, *a5, 4, A16, A16, A16, A16, None, A16, 2, 4, A16, 16, 1,
                 None) == 6
        assert f(_c(V2), 0, *[None] * 5, 0, *[None] * 6, 1, 1, None, 1, 1, None) == 0


def test_q4_entry_errors(L):
    assert L.mla_cache_q4_bytes_per_token(_c(V2)) == 304             # 576 / 2 + 16
    assert L.mla_cache_q4_bytes_per_token(_c(TINY)) == 0             # D = 80: not a multiple of 32
    ok = mla.Config(num_heads=4, kv_rank=112, rope_dim=16, nope_dim=32, v_dim=32, dtype=mla.F32)
    assert L.mla_cache_q4_bytes_per_token(_c(ok)) == 80               # 128 / 2 + 16
    odd = mla.Config(num_heads=4, kv_rank=64, rope_dim=8, nope_dim=32, v_dim=32, dtype=mla.F32)
    assert L.mla_cache_q4_bytes_per_token(_c(odd)) == 0              # D = 72: not a multiple of 32
    def dec(cfg=V2, q_len=1, batch=2, S=4, tree=None, o=A16):
        return L.mla_decode_paged_q4(_c(cfg), batch, q_len, 0, S, 256, A16, A16, 8, A16, 4,
                                     A16, tree, o, A16, None)
    assert dec(o=None) == 1 and dec(tree=MIS) == 4 and dec(q_len=65, tree=A16) == 2
    assert dec(cfg=mla.Config(num_heads=8)) == 6 and dec(cfg=TINY) == 6
    assert dec(batch=0) == 0
    args = [A16, A16, A16, A16]
    assert L.mla_cache_append_q4(_c(V2), 8, *args, MIS, A16, 2, 4, A16, 16, 1, None) == 4
    assert L.mla_cache_append_q4(_c(V2), 8, *args, None, A16, 2, 4, None, 16, 1, None) == 1
    assert L.mla_cache_append_q4(_c(odd), 8, *args, None, A16, 2, 4, A16, 16, 1, None) == 6


def test_sparse_entry_errors(L):
    c = _c(V2)
    # indexer key append: width rule, pointers, alignment, empty call
    assert L.mla_index_append(c, 130, 4, A16, A16, A16, A16, 2, 4, A16, 16, None) == 2
    assert L.mla_index_append(c, 128, 4, None, A16, A16, A16, 2, 4, A16, 16, None) == 1
    assert L.mla_index_append(c, 128, 4, A16, A16, MIS, A16, 2, 4, A16, 16, None) == 4
    assert L.mla_index_append(c, 128, 0, None, None, None, None, 2, 4, None, 16, None) == 0
    # index scores: heads range, ld below max_seq_len, capacity, unsupported LDS size
    def sc(heads=64, dim=128, ld=256, max_len=256, max_pages=4, scores=A16, cfg=V2):
        return L.mla_index_scores(_c(cfg), heads, dim, 2, 1, max_len, A16, A16, A16, 8, A16,
                                  max_pages, A16, scores, ld, None)
    assert sc(heads=0) == 2 and sc(heads=257) == 2
    assert sc(ld=255) == 2
    assert sc(max_len=300) == 5                                     # 4 pages x 64 < 300
    assert sc(scores=None) == 1 and sc(scores=MIS) == 4
    assert sc(heads=256, dim=1024, cfg=TINY) == 6                   # generic needs > 160 KiB
    # top-k
    assert L.mla_topk_select(2, 1, 256, 0, A16, 256, A16, A16, A16, A16, None) == 2
    assert L.mla_topk_select(2, 1, 256, 65537, A16, 256, A16, A16, A16, A16, None) == 2
    assert L.mla_topk_select(2, 1, 256, 64, A16, 200, A16, A16, A16, A16, None) == 2
    assert L.mla_topk_select(2, 1, 256, 64, A16, 256, A16, A16, None, A16, None) == 1
    assert L.mla_topk_select(2, 1, 256, 64, A16, 256, A16, None, A16, A16, None) == 1
    assert L.mla_topk_select(2, 1, 256, 64, A16, 256, A16, MIS, A16, A16, None) == 4
    assert L.mla_topk_select(0, 1, 256, 64, None, 256, None, None, None, None, None) == 0
    assert L.mla_topk_workspace_bytes(8, 1) == 8 * 4100 * 4
    # index scores + top-k in one call: the union of both calls' checks
    def st(heads=64, topk=64, ld=256, max_len=256, ws=A16, cfg=V2):
        return L.mla_index_scores_topk(_c(cfg), heads, 128, 2, 1, max_len, A16, A16, A16, 8, A16,
                                       4, A16, A16, ld, topk, ws, A16, A16, None)
    assert st(heads=0) == 2 and st(topk=0) == 2 and st(topk=65537) == 2
    assert st(ld=255) == 2 and st(max_len=300) == 5
    assert st(ws=None) == 1 and st(ws=MIS) == 4
    assert L.mla_topk_workspace_bytes(0, 1) == 0 and L.mla_topk_workspace_bytes(2, 0) == 0
    # sparse decode
    def dec(topk=2048, S=16, counts=A16, batch=2):
        return L.mla_decode_sparse(c, batch, 1, topk, S, 256, A16, A16, 8, A16, 4, A16, A16,
                                   counts, A16, A16, None)
    assert dec(topk=0) == 2 and dec(S=0) == 2
    assert dec(counts=None) == 1 and dec(counts=MIS) == 4
    assert dec(batch=0) == 0


def test_sparse_chunk_and_kernel_choice(L):
    assert mla.sparse_chunk(2048, 16) == 128
    assert mla.sparse_chunk(2048, 3) == 704                # ceil(2048/3) = 683 -> 704
    assert mla.sparse_chunk(100, 1) == 128
    assert mla.sparse_chunk(0, 4) == 0 and mla.sparse_chunk(64, 0) == 0
    assert mla.decode_sparse_kernel_kind(V2, 2048, 16) == "mfma_rows16_gather"
    assert mla.decode_sparse_kernel_kind(V2, 2048, 2) == "mfma_rows16_gather"  # chunk 1024
    assert mla.decode_sparse_kernel_kind(V2, 2048, 1) == "generic_gather"      # chunk > 1,984
    assert mla.decode_sparse_kernel_kind(mla.Config(num_heads=8), 2048, 16) == "generic_gather"
    assert mla.decode_sparse_kernel_kind(mla.Config(num_heads=128), 2048, 16) == \
        "mfma_rows16_gather"
    assert mla.decode_sparse_kernel_kind(TINY, 64, 2) == "generic_gather"
    assert mla.decode_sparse_kernel_kind(V2, 0, 2) == "invalid"
