"""Seeded generator: determinism, shapes, value recipe and page-table structure."""
import numpy as np

import workload


def test_same_seed_same_bytes():
    wl = workload.WORKLOADS["v2lite_paged_varlen"].replace(batch=4, len_range=(1, 300))
    a, b = workload.make(wl, 3), workload.make(wl, 3)
    for name in ["seq_lens", "w_uk", "w_uv", "q_nope", "q_rope", "c", "k_rope", "page_table"]:
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c = workload.make(wl, 4)
    assert not np.array_equal(a.q_nope, c.q_nope)


def test_lengths_in_range_and_page_table_is_a_permutation():
    wl = workload.WORKLOADS["v2lite_paged_varlen"]
    inp = workload.make(wl, 0, with_latents=False)
    assert inp.seq_lens.min() >= 1024 and inp.seq_lens.max() <= 32768
    npg = -(-inp.seq_lens // 64)
    assert inp.num_pages == int(npg.sum())
    used = np.concatenate([inp.page_table[b, :n] for b, n in enumerate(npg)])
    assert np.array_equal(np.sort(used), np.arange(inp.num_pages))
    assert not np.array_equal(used, np.arange(inp.num_pages))       # really permuted
    for b, n in enumerate(npg):
        assert np.all(inp.page_table[b, n:] == -1)


def test_identity_layout_for_contiguous_workloads():
    wl = workload.WORKLOADS["v2lite_32k"]
    inp = workload.make(wl, 0, with_latents=False)
    assert np.array_equal(inp.page_table.reshape(-1), np.arange(8 * 512))


def test_bf16_rounding_is_nearest_even_and_values_representable():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e-3], dtype=np.float32)
    r = workload.round_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0 + 2 ** -7)
    assert r[3] == -2.5
    bits = workload.bf16_bits(r)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, r)
    wl = workload.WORKLOADS["v2lite_32k"].replace(batch=1, seq_len=64)
    inp = workload.make(wl, 0)
    for arr in (inp.c, inp.w_uk, inp.q_nope):
        assert np.array_equal(workload.round_bf16(arr), arr)


def test_value_recipe():
    wl = workload.WORKLOADS["v2lite_32k"].replace(batch=2, seq_len=4096)
    inp = workload.make(wl, 0)
    assert abs(inp.c.std() - 1.0) < 0.01 and abs(inp.c.mean()) < 0.01
    assert abs(inp.w_uk.std() * np.sqrt(512) - 1.0) < 0.02
    assert abs(inp.q_rope.std() - 1.0) < 0.1


def test_sequence_streams_are_independent():
    wl = workload.WORKLOADS["v2lite_paged_varlen"].replace(batch=3, len_range=(10, 50))
    inp = workload.make(wl, 1)
    c1, k1 = workload.seq_latents(wl, 1, 1, int(inp.seq_lens[1]))
    s, e = inp.offsets[1], inp.offsets[2]
    assert np.array_equal(c1, inp.c[s:e]) and np.array_equal(k1, inp.k_rope[s:e])
