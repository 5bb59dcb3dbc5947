"""GPU parity of chunked prefill, through the C ABI.

Chunked prefill ("Beyond the Attention Bottleneck", "Chunked Prefilling"):
the prompt enters the cache chunk by chunk and each chunk's queries attend
causally to the cache as it then stands. In the absorbed form a chunk of C
tokens is one step of the library with q_len = C: absorb + append of the
chunk's rows, the decode with the chain mask (query i at position P + i sees
t <= P + i; a block stops streaming after the last token its rows see), then
merge and up-projection. The chunks of a prompt run one after another on a
cache that only the steps themselves fill, and every chunk's outputs are
compared with oracle.prefill_in_chunks under the bf16 bounds (max|err| <=
1e-2 max|ref|, lse within 1e-2; 1e-4 / 1e-5 for fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import workload
import mla_latent_kv_03_amd as mla
from mla_latent_kv_03_amd.pipeline import DecodeStep, fill_cache, upload

from gpu_case import assert_close, lse_atol, poisoned_pool, tau, to64

pytestmark = pytest.mark.gpu

W = workload.WORKLOADS


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


def _prefill(wl, chunk, cached=0, seed=3, num_splits=1):
    """Run the prompt of every sequence (wl.seq_len tokens) through the
    device chunk by chunk; returns per-chunk device outputs and the inputs."""
    N = wl.seq_len
    inp = workload.make(wl.replace(q_len=N), seed)
    cfg = mla.Config.from_workload(wl)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    B = wl.batch
    pool = poisoned_pool(cfg, inp.num_pages)
    pt = upload(inp.page_table, torch.int32)
    c_all = inp.c.reshape(B, N, -1)
    k_all = inp.k_rope.reshape(B, N, -1)
    if cached:  # the prefix already in the cache
        si = np.repeat(np.arange(B, dtype=np.int32), cached)
        pos = np.tile(np.arange(cached, dtype=np.int32), B)
        fill_cache(cfg, pool, pt, upload(c_all[:, :cached].reshape(B * cached, -1), dt),
                   upload(k_all[:, :cached].reshape(B * cached, -1), dt),
                   upload(si, torch.int32), upload(pos, torch.int32))
    w_uk, w_uv = upload(inp.w_uk, dt), upload(inp.w_uv, dt)
    kinds, outs = [], []
    for s in range(cached, N, chunk):
        e = min(N, s + chunk)
        C = e - s
        lens = np.full(B, e, np.int32)
        step = DecodeStep(cfg, B, C, num_splits, lens)
        kinds.append(mla.decode_kernel_kind(cfg, C))
        step.run(upload(np.ascontiguousarray(inp.q_nope[:, s:e]), dt),   # queries of tokens s..e-1
                 upload(np.ascontiguousarray(inp.q_rope[:, s:e]), dt),
                 w_uk, w_uv,
                 upload(np.ascontiguousarray(c_all[:, s:e]).reshape(B * C, -1), dt),
                 upload(np.ascontiguousarray(k_all[:, s:e]).reshape(B * C, -1), dt),
                 pool, pt, upload(lens, torch.int32))
        torch.cuda.synchronize()
        outs.append({"o": to64(step.out), "o_lat": to64(step.o_lat), "lse": to64(step.lse)})
    return inp, outs, kinds


def _check(wl, inp, outs, chunk, cached):
    N = wl.seq_len
    for b in range(wl.batch):
        c, kr = inp.seq(b)
        ref = oracle.prefill_in_chunks(c, kr, inp.q_nope[b][cached:], inp.q_rope[b][cached:],
                                       inp.w_uk, inp.w_uv, wl.softmax_scale, chunk,
                                       wl.rope_base, cached=cached)
        got = {k: np.concatenate([o[k][b] for o in outs]) for k in ("o", "o_lat", "lse")}
        assert_close(got["o"], ref[0], tau(wl), f"seq {b} o")
        assert_close(got["o_lat"], ref[1], tau(wl), f"seq {b} o_lat")
        assert_close(got["lse"], ref[2], lse_atol(wl), f"seq {b} lse", lse=True)


PREFILL = {  # name: (workload, chunk, cached prefix, kernels expected among the chunks)
    "v2lite_chunks_256": (W["v2lite_32k"].replace(batch=2, seq_len=700, paged=True), 256, 0,
                          {"mfma_ws"}),
    "v2lite_after_prefix": (W["v2lite_32k"].replace(batch=2, seq_len=900, paged=True), 128, 333,
                            {"mfma_ws", "mfma_rows16"}),  # last chunk: 55 x 16 rows
    "v2lite_odd_chunks": (W["v2lite_32k"].replace(batch=1, seq_len=150, paged=True), 7, 0,
                          {"mfma_rows16", "mfma_ws"}),
    "h128_chunks": (W["v2_h128_8k"].replace(batch=1, seq_len=400), 160, 0, {"mfma_ws"}),
    "tiny_f32_chunks": (W["tiny_f32"].replace(batch=2, seq_len=200, paged=True), 48, 0,
                        {"generic"}),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_chunked_prefill_matches_oracle(name):
    wl, chunk, cached, kinds = PREFILL[name]
    inp, outs, got_kinds = _prefill(wl, chunk, cached)
    assert set(got_kinds) <= kinds | {"generic"} and set(got_kinds) & kinds, got_kinds
    _check(wl, inp, outs, chunk, cached)


def test_chunked_prefill_with_split_partitions():
    # the same chunks through four partitions per sequence (the merge must
    # drop the partitions a chunk's queries cannot see)
    wl, chunk, cached, _ = PREFILL["v2lite_chunks_256"]
    inp, outs, _ = _prefill(wl, chunk, cached, num_splits=4)
    _check(wl, inp, outs, chunk, cached)


def test_full_size_last_chunk_of_32k_prompt_sampled():
    wl = W["v2lite_prefill_32k_c4k"]
    inp = workload.make(wl, 0)
    cfg = mla.Config.from_workload(wl)
    dt = torch.bfloat16
    L, C, H = wl.seq_len, wl.q_len, wl.heads
    P = L - C
    pool = poisoned_pool(cfg, inp.num_pages)
    pt = upload(inp.page_table, torch.int32)
    fill_cache(cfg, pool, pt, upload(inp.c[:P], dt), upload(inp.k_rope[:P], dt),
               upload(np.zeros(P, np.int32), torch.int32),
               upload(np.arange(P, dtype=np.int32), torch.int32))
    step = DecodeStep(cfg, 1, C, 1, inp.seq_lens)
    assert mla.decode_kernel_kind(cfg, C) == "mfma_ws"
    step.run(upload(inp.q_nope, dt), upload(inp.q_rope, dt), upload(inp.w_uk, dt),
             upload(inp.w_uv, dt), upload(inp.c[P:], dt), upload(inp.k_rope[P:], dt), pool, pt,
             upload(inp.seq_lens, torch.int32))
    torch.cuda.synchronize()
    got = {"o": to64(step.out), "o_lat": to64(step.o_lat), "lse": to64(step.lse)}
    hs = [0, 9, 15]
    w_uk, w_uv = inp.w_uk[hs], inp.w_uv[hs]
    for j in (0, 1, 777, 2048, C - 1):
        # query j at position P + j: a one-token decode over tokens 0 .. P + j
        o, ol, lse = oracle.attend_sequence(inp.c[:P + j + 1], inp.k_rope[:P + j + 1],
                                            inp.q_nope[0][j:j + 1][:, hs],
                                            inp.q_rope[0][j:j + 1][:, hs],
                                            w_uk, w_uv, wl.softmax_scale, wl.rope_base)
        assert_close(got["o"][0, j][hs], o[0], tau(wl), f"query {j} o")
        assert_close(got["o_lat"][0, j][hs], ol[0], tau(wl), f"query {j} o_lat")
        assert_close(got["lse"][0, j][hs], lse[0], lse_atol(wl), f"query {j} lse", lse=True)


# ---------------------------------------------------------------- unabsorbed form
# mla_prefill_unabsorbed expands every cached latent into per-head keys and
# values ("Down-Projection and Up-Projection Mechanics") and runs dense causal
# attention per head; its output (value space) and lse are the same attention
# as the absorbed form's (the oracle's o and lse), under the same bounds.
def _prefill_unabsorbed(wl, chunk, cached=0, seed=3):
    N = wl.seq_len
    inp = workload.make(wl.replace(q_len=N), seed)
    cfg = mla.Config.from_workload(wl)
    dt = torch.bfloat16
    B, H = wl.batch, wl.heads
    pool = poisoned_pool(cfg, inp.num_pages)
    pt = upload(inp.page_table, torch.int32)
    c_all = inp.c.reshape(B, N, -1)
    k_all = inp.k_rope.reshape(B, N, -1)
    if cached:
        si = np.repeat(np.arange(B, dtype=np.int32), cached)
        pos = np.tile(np.arange(cached, dtype=np.int32), B)
        fill_cache(cfg, pool, pt, upload(c_all[:, :cached].reshape(B * cached, -1), dt),
                   upload(k_all[:, :cached].reshape(B * cached, -1), dt),
                   upload(si, torch.int32), upload(pos, torch.int32))
    w_uk, w_uv = upload(inp.w_uk, dt), upload(inp.w_uv, dt)
    outs = []
    for s in range(cached, N, chunk):
        e = min(N, s + chunk)
        C = e - s
        si = np.repeat(np.arange(B, dtype=np.int32), C)
        pos = np.tile(np.arange(s, e, dtype=np.int32), B)
        mla.cache_append(cfg, upload(np.ascontiguousarray(c_all[:, s:e]).reshape(B * C, -1), dt),
                         upload(np.ascontiguousarray(k_all[:, s:e]).reshape(B * C, -1), dt),
                         upload(si, torch.int32), upload(pos, torch.int32), pt, pool,
                         mla.APPEND_ROTATE)
        res = {"o": [], "lse": []}
        for b in range(B):
            ws = torch.empty(mla.prefill_workspace_bytes(cfg, e, C), dtype=torch.uint8,
                             device="cuda")
            out = torch.empty((C, H, wl.v_dim), dtype=dt, device="cuda")
            lse = torch.empty((C, H), dtype=torch.float32, device="cuda")
            mla.prefill_unabsorbed(cfg, upload(np.ascontiguousarray(inp.q_nope[b, s:e]), dt),
                                   upload(np.ascontiguousarray(inp.q_rope[b, s:e]), dt), w_uk,
                                   w_uv, pool, pt[b], e, ws, out, lse)
            torch.cuda.synchronize()
            res["o"].append(to64(out))
            res["lse"].append(to64(lse))
        outs.append({k: np.stack(v) for k, v in res.items()})
    return inp, outs


UNABSORBED = {  # name: (workload, chunk, cached prefix)
    "v2lite_chunks_256": (W["v2lite_32k"].replace(batch=2, seq_len=700, paged=True), 256, 0),
    "v2lite_after_prefix": (W["v2lite_32k"].replace(batch=2, seq_len=900, paged=True), 129, 333),
    "v2lite_odd_chunks": (W["v2lite_32k"].replace(batch=1, seq_len=150, paged=True), 7, 0),
    "h128_chunks": (W["v2_h128_8k"].replace(batch=1, seq_len=400), 160, 0),
    "page16": (W["v2lite_paged_varlen"].replace(batch=1, seq_len=500, len_range=None,
                                                page_size=16), 300, 0),
}


@pytest.mark.parametrize("name", list(UNABSORBED))
def test_unabsorbed_prefill_matches_oracle(name):
    wl, chunk, cached = UNABSORBED[name]
    inp, outs = _prefill_unabsorbed(wl, chunk, cached)
    for b in range(wl.batch):
        c, kr = inp.seq(b)
        ref = oracle.prefill_in_chunks(c, kr, inp.q_nope[b][cached:], inp.q_rope[b][cached:],
                                       inp.w_uk, inp.w_uv, wl.softmax_scale, chunk,
                                       wl.rope_base, cached=cached)
        got_o = np.concatenate([o["o"][b] for o in outs])
        got_l = np.concatenate([o["lse"][b] for o in outs])
        assert_close(got_o, ref[0], tau(wl), f"seq {b} o")
        assert_close(got_l, ref[2], lse_atol(wl), f"seq {b} lse", lse=True)


def test_unabsorbed_form_choice_and_errors():
    cfg = mla.Config(num_heads=16)
    assert mla.prefill_form(cfg, 4096, 32768) == "unabsorbed"
    assert mla.prefill_form(cfg, 64, 32768) == "absorbed"
    assert mla.prefill_form(cfg, 1023, 32768) == "absorbed"
    assert mla.prefill_form(mla.Config(num_heads=4, kv_rank=64, rope_dim=16, nope_dim=32,
                                       v_dim=32, dtype=mla.F32), 4096, 8192) == "absorbed"
    assert mla.prefill_workspace_bytes(cfg, 1000, 2000) == 0


def test_full_size_last_chunk_unabsorbed_sampled():
    wl = W["v2lite_prefill_32k_c4k"]
    inp = workload.make(wl, 0)
    cfg = mla.Config.from_workload(wl)
    dt = torch.bfloat16
    L, C, H = wl.seq_len, wl.q_len, wl.heads
    P = L - C
    pool = poisoned_pool(cfg, inp.num_pages)
    pt = upload(inp.page_table, torch.int32)
    fill_cache(cfg, pool, pt, upload(inp.c, dt), upload(inp.k_rope, dt),
               upload(np.zeros(L, np.int32), torch.int32),
               upload(np.arange(L, dtype=np.int32), torch.int32))
    assert mla.prefill_form(cfg, C, L) == "unabsorbed"
    ws = torch.empty(mla.prefill_workspace_bytes(cfg, L, C), dtype=torch.uint8, device="cuda")
    out = torch.empty((C, H, wl.v_dim), dtype=dt, device="cuda")
    lse = torch.empty((C, H), dtype=torch.float32, device="cuda")
    mla.prefill_unabsorbed(cfg, upload(inp.q_nope[0], dt), upload(inp.q_rope[0], dt),
                           upload(inp.w_uk, dt), upload(inp.w_uv, dt), pool, pt[0], L, ws, out, lse)
    torch.cuda.synchronize()
    got_o, got_l = to64(out), to64(lse)
    hs = [0, 9, 15]
    w_uk, w_uv = inp.w_uk[hs], inp.w_uv[hs]
    for j in (0, 1, 777, 2048, C - 1):
        o, ol, l_ = oracle.attend_sequence(inp.c[:P + j + 1], inp.k_rope[:P + j + 1],
                                           inp.q_nope[0][j:j + 1][:, hs],
                                           inp.q_rope[0][j:j + 1][:, hs],
                                           w_uk, w_uv, wl.softmax_scale, wl.rope_base)
        assert_close(got_o[j][hs], o[0], tau(wl), f"query {j} o")
        assert_close(got_l[j][hs], l_[0], lse_atol(wl), f"query {j} lse", lse=True)
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
