"""GPU parity of the sparse read, through the C ABI.

The sparse read ("DeepSeek's Config Says 16 KV Heads, Its Cache Holds a Ninth
of That", section 6, "Sparse attention"): mla_index_scores rates every cached
token, mla_topk_select keeps the best topk each query sees, mla_decode_sparse
attends over those tokens only. Checked against the oracle on the same seeded
inputs:
  * top-k alone on seeded fp32 score rows (ties, -0/+0, -inf): the selected
    index lists and counts bit-exact (both sides decide on the same fp32
    values), LDS-resident and streamed sequence lengths;
  * index scores: each within its own fp32 error bound (the standard bound
    for a sum in any order: gamma_n = n u / (1 - n u), u = 2^-24, times the
    sum of the absolute terms, for the dot products and the head sum);
  * the sparse decode alone over seeded random selections: the bf16 bounds
    of the dense decode (max|err| <= 1e-2 max|ref|, lse within 1e-2), every
    kernel class;
  * the whole step on exact-score inputs (integer indexer queries and keys,
    head weights in steps of 1/8: every score exact in fp32): the selected
    tokens bit-exact against the oracle's, ties included, then the outputs;
  * the whole step at full size with N(0, 1) indexer inputs, where the
    boundary holds near-ties that fp32 rounding may order either way: the
    selection is checked to be a valid top-k under the per-token error bound
    (sized, visible, no excluded token provably above an included one), the
    outputs against the oracle's own selection within the bf16 bounds.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
import mla_latent_kv_03_amd as mla
from mla_latent_kv_03_amd.pipeline import upload

from gpu_case import Case, check_against_oracle, poisoned_index_pool, to64

pytestmark = pytest.mark.gpu

W = workload.WORKLOADS


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


# ---------------------------------------------------------------- top-k alone
def _topk_gpu(scores, lens, Q, K, max_len):
    B = len(lens)
    sc = upload(scores.reshape(B, Q, -1), torch.float32)
    sl = upload(np.asarray(lens, np.int32), torch.int32)
    idx = torch.full((B, Q, K), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Q), -9, dtype=torch.int32, device="cuda")
    ws = torch.zeros(mla.topk_workspace_bytes(B, Q), dtype=torch.uint8, device="cuda")
    mla.topk_select(sc, sl, idx, cnt, max_len, ws)
    mla.topk_select(sc, sl, idx, cnt, max_len, ws)   # a second call on the same workspace
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0, "the workspace must be left all zero"
    return idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("length,K,Q", [(100, 7, 1), (3000, 256, 2), (32768, 2048, 1),
                                        (40000, 2048, 1), (5000, 4999, 1), (700, 2048, 3),
                                        (1024, 1, 1)])
def test_topk_matches_oracle_bit_exact(length, K, Q):
    B = 3
    lens = [length, max(Q, length - 37), max(Q, length // 3)]
    rows = workload.score_rows(11, B * Q, length).reshape(B, Q, length)
    idx, cnt = _topk_gpu(rows, lens, Q, K, length)
    for b in range(B):
        for j in range(Q):
            vis = lens[b] - Q + j + 1
            want = oracle.topk_tokens(rows[b, j], K, vis)
            assert cnt[b, j] == len(want), (b, j)
            assert idx[b, j, :len(want)].tolist() == want.tolist(), (b, j)


def test_topk_special_values_and_invalid_sequences():
    L, K = 600, 50
    rows = workload.score_rows(12, 5, L, ties=False)
    rows[0] = 1.0                              # all equal: the first K tokens
    rows[1, ::2] = -np.inf                     # half -inf
    rows[2, :] = np.where(np.arange(L) % 3 == 0, -0.0, 0.0)  # signed zeros only
    rows[3, 17] = np.nan                       # NaN: sequence reported invalid
    fmax = np.finfo(np.float32).max            # keys over nearly the whole 32-bit range
    rows[4, ::7] = np.inf
    rows[4, 1::7] = -np.inf
    rows[4, 2::7] = fmax
    rows[4, 3::7] = -fmax
    rows[4, 4::7] = np.float32(1e-40)          # denormals
    idx, cnt = _topk_gpu(rows, [L] * 5, 1, K, L)
    for b in (0, 1, 2, 4):
        want = oracle.topk_tokens(rows[b], K, L)
        assert cnt[b, 0] == K and idx[b, 0, :K].tolist() == want.tolist()
    want = oracle.topk_tokens(rows[4], 150, L)           # the cut inside the +-FLT_MAX copies
    idx4, cnt4 = _topk_gpu(rows[4:5], [L], 1, 150, L)
    assert cnt4[0, 0] == 150 and idx4[0, 0].tolist() == want.tolist()
    assert cnt[3, 0] == -1 and np.all(idx[3] == -7)
    # lengths outside [Q, max_seq_len]
    idx, cnt = _topk_gpu(rows[:2], [L + 1, 0], 1, K, L)
    assert cnt.tolist() == [[-1], [-1]]


def test_topk_crowded_bin_reads_every_score():
    # 20,000 scores in one coarse bin (same sign, exponent and top mantissa
    # bits): more than the gathered-key array holds, so the narrowing reads
    # every score; one row of equal values, one spread inside [1, 1.125)
    L, K = 20000, 777
    rng = np.random.default_rng(3)
    rows = np.empty((2, L), np.float32)
    rows[0] = 1.0
    rows[1] = (1.0 + rng.integers(0, 1 << 17, L) * 2.0 ** -20).astype(np.float32)
    idx, cnt = _topk_gpu(rows, [L, L], 1, K, L)
    for b in range(2):
        want = oracle.topk_tokens(rows[b], K, L)
        assert cnt[b, 0] == K and idx[b, 0].tolist() == want.tolist()


# ---------------------------------------------------------------- index scores
U32 = 2.0 ** -24


def _gamma(n):
    return n * U32 / (1 - n * U32)


def _scores_and_bound(inp, b, j, n):
    """fp64 scores of tokens 0..n-1 for query j, and the bound on the error of
    any fp32 evaluation: dot products and head sum each within gamma of the
    sum of their absolute terms (the inputs themselves are exact)."""
    q = np.asarray(inp.q_idx[b][j], np.float64)
    w = np.asarray(inp.w_idx[b][j], np.float64)
    k = np.asarray(inp.seq_index_keys(b)[:n], np.float64)
    dots = q @ k.T
    s = w @ np.maximum(dots, 0.0)
    eps = (np.abs(w) @ (np.abs(q) @ np.abs(k).T)) * _gamma(q.shape[1]) * (1 + _gamma(q.shape[0])) \
        + _gamma(q.shape[0]) * (np.abs(w) @ np.maximum(dots, 0.0))
    return s, eps + 1e-30


def _index_case(wl, seed, lens):
    inp = workload.make(wl, seed, seq_lens=lens)
    cfg = mla.Config.from_workload(wl)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    pool = poisoned_index_pool(cfg, inp.num_pages, wl.index_dim)
    pt = upload(inp.page_table, torch.int32)
    si = np.concatenate([np.full(int(L), b, np.int32) for b, L in enumerate(inp.seq_lens)])
    pos = np.concatenate([np.arange(int(L), dtype=np.int32) for L in inp.seq_lens])
    mla.index_append(cfg, upload(inp.k_idx, dt), upload(si, torch.int32),
                     upload(pos, torch.int32), pt, pool)
    return inp, cfg, dt, pool, pt


INDEX_SHAPES = {
    "mfma_64x128": (W["v2lite_32k_dsa"].replace(batch=3, seq_len=None, len_range=(1, 1500),
                                                paged=True, q_len=2), [1500, 1023, 2]),
    "generic_f32": (W["tiny_f32"].replace(batch=2, q_len=2, seq_len=300, index_topk=50,
                                          index_heads=4, index_dim=8, paged=True), None),
    "generic_bf16_32x64": (W["v2lite_32k_dsa"].replace(batch=2, seq_len=700, paged=True,
                                                       index_heads=32, index_dim=64), None),
}


@pytest.mark.parametrize("name", list(INDEX_SHAPES))
def test_index_scores_match_oracle(name):
    wl, lens = INDEX_SHAPES[name]
    inp, cfg, dt, pool, pt = _index_case(wl, 3, lens)
    B, Q, L = wl.batch, wl.q_len, wl.max_seq_len
    sc = torch.full((B, Q, L + 5), 123.0, dtype=torch.float32, device="cuda")
    mla.index_scores(cfg, upload(np.ascontiguousarray(inp.q_idx), dt),
                     upload(np.ascontiguousarray(inp.w_idx), torch.float32), pool, pt,
                     upload(inp.seq_lens, torch.int32), sc, L)
    torch.cuda.synchronize()
    got = sc.cpu().numpy().astype(np.float64)
    for b in range(B):
        Lb = int(inp.seq_lens[b])
        for j in range(Q):
            ref, eps = _scores_and_bound(inp, b, j, Lb)
            err = np.abs(got[b, j, :Lb] - ref)
            assert np.all(err <= eps), (b, j, float((err / eps).max()))
        assert np.all(got[b, :, Lb:] == 123.0)   # nothing past the sequence is written


def test_index_scores_invalid_page_is_nan():
    wl, lens = INDEX_SHAPES["mfma_64x128"]
    inp, cfg, dt, pool, pt = _index_case(wl, 4, lens)
    pt_bad = pt.clone()
    pt_bad[0, 3] = inp.num_pages + 5     # tokens 192..255 of sequence 0
    B, Q, L = wl.batch, wl.q_len, wl.max_seq_len
    sc = torch.zeros((B, Q, L), dtype=torch.float32, device="cuda")
    mla.index_scores(cfg, upload(np.ascontiguousarray(inp.q_idx), dt),
                     upload(np.ascontiguousarray(inp.w_idx), torch.float32), pool, pt_bad,
                     upload(inp.seq_lens, torch.int32), sc, L)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    assert np.all(np.isnan(got[0, :, 192:256])) and np.all(np.isfinite(got[0, :, :192]))
    assert np.all(np.isfinite(got[1, :, :int(inp.seq_lens[1])]))


@pytest.mark.parametrize("name", ["mfma_64x128", "generic_f32"])
def test_index_scores_topk_equals_the_two_calls(name):
    # mla_index_scores_topk: the same scores bit for bit and the same selection
    # as mla_index_scores followed by mla_topk_select, on ragged lengths, an
    # invalid length and a token whose page entry is invalid (NaN score: the
    # sequence reported invalid); the workspace is left all zero
    wl, lens = INDEX_SHAPES[name]
    inp, cfg, dt, pool, pt = _index_case(wl, 5, lens)
    B, Q, L = wl.batch, wl.q_len, wl.max_seq_len
    K = min(wl.index_topk, 300)
    pt_bad = pt.clone()
    pt_bad[B - 1, 0] = inp.num_pages + 3               # the last sequence's first page
    seq_lens = inp.seq_lens.copy()
    seq_lens[0] = L + 1 if B > 2 else seq_lens[0]      # beyond max_seq_len: invalid
    sl = upload(seq_lens, torch.int32)
    q_idx = upload(np.ascontiguousarray(inp.q_idx), dt)
    w_idx = upload(np.ascontiguousarray(inp.w_idx), torch.float32)
    out = []
    for fused in (False, True):
        sc = torch.full((B, Q, L + 3), 7.0, dtype=torch.float32, device="cuda")
        idx = torch.full((B, Q, K), -5, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Q), -9, dtype=torch.int32, device="cuda")
        ws = torch.zeros(mla.topk_workspace_bytes(B, Q), dtype=torch.uint8, device="cuda")
        for _ in range(2):  # a second call on the same workspace
            if fused:
                mla.index_scores_topk(cfg, q_idx, w_idx, pool, pt_bad, sl, sc, L, idx, cnt, ws)
            else:
                mla.index_scores(cfg, q_idx, w_idx, pool, pt_bad, sl, sc, L)
                mla.topk_select(sc, sl, idx, cnt, L, ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
        out.append((sc.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()))
    (s0, i0, c0), (s1, i1, c1) = out
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
    assert np.array_equal(c0, c1) and np.array_equal(i0, i1)
    assert np.all(c1[B - 1] == -1)                       # NaN among the visible scores
    if B > 2:
        assert np.all(c1[0] == -1)                       # invalid length
    assert np.any(c1 > 0)


# ---------------------------------------------------------------- sparse decode alone
def _random_selection(inp, K, seed):
    wl = inp.wl
    return [[workload.random_selection(seed, b, j, int(inp.seq_lens[b]) - wl.q_len + j + 1, K)
             for j in range(wl.q_len)] for b in range(wl.batch)]


def _upload_selection(sel, B, Q, K):
    idx = np.full((B, Q, K), -1, np.int32)
    cnt = np.zeros((B, Q), np.int32)
    for b in range(B):
        for j in range(Q):
            idx[b, j, :len(sel[b][j])] = sel[b][j]
            cnt[b, j] = len(sel[b][j])
    return upload(idx, torch.int32), upload(cnt, torch.int32)


SPARSE = {  # name: (workload, num_splits, expected kernel)
    "v2lite_gather": (W["v2lite_32k_dsa"].replace(batch=3, seq_len=None, len_range=(1, 5000),
                                                  paged=True, index_topk=700), 4,
                      "mfma_rows16_gather"),
    "v2lite_q3_gather": (W["v2lite_32k_dsa"].replace(batch=2, q_len=3, seq_len=2500, paged=True,
                                                     index_topk=512), 8, "mfma_rows16_gather"),
    "h128_gather": (W["v2_h128_8k"].replace(batch=2, seq_len=3000, index_topk=400), 3,
                    "mfma_rows16_gather"),
    "one_split_generic": (W["v2lite_32k_dsa"].replace(batch=2, seq_len=3000, paged=True,
                                                      index_topk=2048), 1, "generic_gather"),
    "tiny_f32_generic": (W["tiny_f32"].replace(batch=3, q_len=2, seq_len=None, len_range=(2, 256),
                                               paged=True, index_topk=60, index_heads=4,
                                               index_dim=8), 3, "generic_gather"),
}


@pytest.mark.parametrize("name", list(SPARSE))
def test_sparse_decode_matches_oracle(name):
    wl, S, kind = SPARSE[name]
    case = Case(wl, seed=5, num_splits=S)
    assert mla.decode_sparse_kernel_kind(case.cfg, wl.index_topk, S) == kind
    sel = _random_selection(case.inp, wl.index_topk, 17)
    st = case.step
    st.indices, st.counts = _upload_selection(sel, wl.batch, wl.q_len, wl.index_topk)
    st.absorb(case.q_nope, case.q_rope, case.w_uk)
    st.decode(case.pool, case.pt, case.seq_lens)
    st.combine_up_project(case.w_uv)
    torch.cuda.synchronize()
    check_against_oracle(case, case.results(), case.oracle(selection=sel))


def test_sparse_decode_invalid_lists_give_nan():
    wl, S, _ = SPARSE["v2lite_gather"]
    case = Case(wl, seed=6, num_splits=S)
    K = wl.index_topk
    sel = _random_selection(case.inp, K, 18)
    st = case.step
    idx, cnt = _upload_selection(sel, wl.batch, wl.q_len, K)
    L0 = int(case.inp.seq_lens[0])
    idx[0, 0, 0] = L0          # past the query's own position
    cnt[1, 0] = K + 1          # count above topk
    st.indices, st.counts = idx, cnt
    st.absorb(case.q_nope, case.q_rope, case.w_uk)
    st.decode(case.pool, case.pt, case.seq_lens)
    st.combine_up_project(case.w_uv)
    torch.cuda.synchronize()
    got = case.results()
    assert np.all(np.isnan(got["lse"][0])) and np.all(np.isnan(got["lse"][1]))
    ref = case.oracle(seqs=[2], selection=sel)
    check_against_oracle(case, got, ref, seqs=[2])


# ---------------------------------------------------------------- the whole step
STEP = {
    "v2lite_step": W["v2lite_32k_dsa"].replace(batch=3, seq_len=None, len_range=(100, 6000),
                                               paged=True, index_topk=1024, index_exact=True),
    "v2lite_q2_step": W["v2lite_32k_dsa"].replace(batch=2, q_len=2, seq_len=4000, paged=True,
                                                  index_topk=300, num_splits=4, index_exact=True),
    "h128_step": W["v2_h128_8k"].replace(batch=2, seq_len=2500, index_topk=512, num_splits=4,
                                         index_exact=True),
    "tiny_f32_step": W["tiny_f32"].replace(batch=2, q_len=2, seq_len=256, index_topk=40,
                                           index_heads=4, index_dim=8, paged=True,
                                           index_exact=True),
}


@pytest.mark.parametrize("name", list(STEP))
def test_sparse_step_matches_oracle(name):
    wl = STEP[name]
    case = Case(wl, seed=7)
    case.run()
    ref = case.oracle()
    idx = case.step.indices.cpu().numpy()
    cnt = case.step.counts.cpu().numpy()
    for b in range(wl.batch):
        for j in range(wl.q_len):
            want = ref["selection"][b][j]
            assert cnt[b, j] == len(want)
            assert idx[b, j, :len(want)].tolist() == want.tolist(), (b, j)
    check_against_oracle(case, case.results(), ref)


@pytest.mark.parametrize("name", ["v2lite_step", "v2lite_q2_step", "h128_step"])
def test_sparse_step_one_launch_append_bit_exact(name):
    """mla_absorb_append_index gives the bits of mla_absorb_append followed by
    mla_index_append: absorbed queries, both caches byte for byte, outputs."""
    wl = STEP[name]
    case = Case(wl, seed=8)
    s = case.step
    case.run(fused=False)
    ref = {k: v.copy() for k, v in case.results().items()}
    ref_q = to64(s.q_full)
    ref_pool = case.pool.view(torch.int16).cpu().numpy().copy()
    ref_ipool = case.index_pool.view(torch.int16).cpu().numpy().copy()
    s.q_full.fill_(float("nan"))
    # poison the rows the step writes, so that a call that wrote nothing shows
    pt, page, Q = case.inp.page_table, wl.page_size, wl.q_len
    for b, L in enumerate(case.inp.seq_lens):
        for t in range(int(L) - Q, int(L)):
            case.pool[int(pt[b, t // page]), t % page].fill_(float("nan"))
            case.index_pool[int(pt[b, t // page]), t % page].fill_(float("nan"))
    case.run(fused=True)
    got = case.results()
    assert np.array_equal(to64(s.q_full), ref_q)
    assert np.array_equal(case.pool.view(torch.int16).cpu().numpy(), ref_pool)
    assert np.array_equal(case.index_pool.view(torch.int16).cpu().numpy(), ref_ipool)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k


def _valid_selection(inp, K, b, j, got):
    """got is a top-K of query j that some fp32 evaluation within the error
    bound could produce: K (or all visible) distinct visible tokens in
    increasing order, and no excluded token provably above an included one.
    Returns the number of tokens where it differs from the fp64 selection."""
    wl = inp.wl
    vis = int(inp.seq_lens[b]) - wl.q_len + j + 1
    n = min(K, vis)
    got = np.asarray(got[:n], np.int64)
    assert len(got) == n and np.all(np.diff(got) > 0) and got[0] >= 0 and got[-1] < vis
    s, eps = _scores_and_bound(inp, b, j, vis)
    m = np.zeros(vis, bool)
    m[got] = True
    if n < vis:
        assert (s[m] + eps[m]).min() >= (s[~m] - eps[~m]).max()
    return int(np.setxor1d(got, oracle.topk_tokens(s, K, vis)).size)


def test_full_size_v2lite_32k_dsa_sampled():
    wl = W["v2lite_32k_dsa"]
    case = Case(wl, seed=0)
    case.run()
    seqs = [0, 5]
    ref = case.oracle(heads=[0, 7, 15], seqs=seqs)
    idx = case.step.indices.cpu().numpy()
    cnt = case.step.counts.cpu().numpy()
    for b in range(wl.batch):
        assert cnt[b, 0] == wl.index_topk
    diffs = [_valid_selection(case.inp, wl.index_topk, b, 0, idx[b, 0]) for b in seqs]
    print(f"tokens whose selection differs from the fp64 one (near-ties): {diffs}")
    check_against_oracle(case, case.results(), ref, heads=[0, 7, 15], seqs=seqs)


def test_index_append_writes_exact_rows():
    wl, lens = INDEX_SHAPES["mfma_64x128"]
    inp, cfg, dt, pool, pt = _index_case(wl, 8, lens)
    got = pool.float().cpu().numpy()
    ptab = inp.page_table
    for b in range(wl.batch):
        keys = inp.seq_index_keys(b)
        for t in (0, int(inp.seq_lens[b]) - 1, int(inp.seq_lens[b]) // 2):
            pg = ptab[b, t // cfg.page_size]
            assert np.array_equal(got[pg, t % cfg.page_size], keys[t]), (b, t)
