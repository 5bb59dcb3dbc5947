"""GPU parity of the 8-bit latent cache, through the C ABI.

mla_cache_append_q8 codes each row's latent part and rotated RoPE part
between their own minimum and maximum ("KV Cache Optimization: Scaling to
Million-Token Contexts", technique 3); mla_decode_paged_q8 attends over the
rows those codes stand for. The append is compared with the oracle's coding
of the same rows (codes bit-exact where the inputs reach both sides
unchanged); the decode step with the fp64 oracle over the decoded rows
(oracle.mla_decode_ref_q8) under the bf16 bounds: max|err| <= 1e-2 * max|ref|,
lse within 1e-2. Unwritten slots of the pool hold 0xFF bytes (NaN minima and
steps), so a slot read past a sequence's end would surface as NaN.
"""
import numpy as np
import pytest
import torch

import oracle
import workload
import mla_latent_kv_03_amd as mla
from mla_latent_kv_03_amd.pipeline import upload

from gpu_case import Case, check_against_oracle, to64

pytestmark = pytest.mark.gpu

W = workload.WORKLOADS


def small(name, **kw):
    return W[name].replace(**kw)


Q8 = {
    "v2lite_q8": small("v2lite_32k_q8", batch=2, seq_len=2048 + 37, num_splits=5),
    "paged_varlen_q8": small("v2lite_paged_varlen", batch=5, len_range=(1, 700), num_splits=3,
                             cache="q8"),
    "q4_chain_q8": small("v2lite_paged_varlen", batch=3, q_len=4, len_range=(4, 900),
                         num_splits=4, cache="q8"),
    "tree_q8": small("v2lite_paged_varlen", batch=3, q_len=5, len_range=(5, 600), num_splits=3,
                     tree="random", cache="q8"),
    "h128_q8": small("v2_h128_8k", batch=2, seq_len=1000, num_splits=3, cache="q8"),
    "chunked_q8": small("v2lite_paged_varlen", batch=6, len_range=(1, 900), num_splits=8,
                        split_chunk=128, cache="q8"),
    "page128_q8": small("v2lite_paged_varlen", batch=3, len_range=(30, 1000), num_splits=5,
                        page_size=128, cache="q8"),
}


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu] {request.node.name}", flush=True)
    yield


@pytest.mark.parametrize("name", list(Q8))
def test_q8_decode_step_matches_oracle(name):
    case = Case(Q8[name], seed=2)
    case.run()
    check_against_oracle(case, case.results(), case.oracle())


@pytest.mark.parametrize("name", ["v2lite_q8", "q4_chain_q8", "tree_q8", "h128_q8"])
def test_q8_absorb_append_one_launch_bit_exact(name):
    """mla_absorb_append_q8 gives the bits of mla_absorb_q followed by
    mla_cache_append_q8: absorbed queries, every byte of the pool, outputs."""
    case = Case(Q8[name], seed=4)
    s = case.step
    case.run(fused=False)
    ref = {k: v.copy() for k, v in case.results().items()}
    ref_q = to64(s.q_full)
    ref_pool = case.pool.cpu().numpy().copy()
    s.q_full.fill_(float("nan"))
    # poison the rows the step writes (the drafted rows' slots), so that a
    # fused call that wrote nothing would show
    pt, page, Q = case.inp.page_table, case.wl.page_size, case.wl.q_len
    for b, L in enumerate(case.inp.seq_lens):
        for t in range(int(L) - Q, int(L)):
            case.pool[int(pt[b, t // page]), t % page].fill_(255)
    case.run(fused=True)
    got = case.results()
    assert np.array_equal(to64(s.q_full), ref_q)
    assert np.array_equal(case.pool.cpu().numpy(), ref_pool)
    for k in ref:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k


@pytest.mark.parametrize("lens,Q", [((1,), 1), ((63, 64, 65), 1), ((4, 128), 4)])
def test_q8_edge_lengths(lens, Q):
    wl = small("v2lite_paged_varlen", batch=len(lens), q_len=Q, len_range=(1, max(lens)),
               num_splits=2, cache="q8")
    case = Case(wl, seed=4, seq_lens=lens)
    case.run()
    check_against_oracle(case, case.results(), case.oracle())


def test_q8_full_size_sampled():
    wl = W["v2lite_32k_q8"]
    case = Case(wl, seed=0)
    case.run()
    got = case.results()
    ref = case.oracle(seqs=[0, 7])
    check_against_oracle(case, got, ref, seqs=[0, 7])
    for k in got:
        assert np.all(np.isfinite(got[k]))


def _pool_rows(pool, inp, wl, seq, pos):
    flat = pool.cpu().numpy().reshape(-1, wl.dim + 16)
    idx = [oracle.cache_slot(inp.page_table, int(s), int(p), wl.page_size) for s, p in zip(seq, pos)]
    return flat[idx]


@pytest.mark.parametrize("mode", [mla.APPEND_RAW, mla.APPEND_ROTATE])
def test_q8_append_codes(mode):
    wl = small("v2lite_paged_varlen", batch=2, len_range=(300, 600), cache="q8")
    inp = workload.make(wl, 8)
    cfg = mla.Config.from_workload(wl)
    rng = np.random.default_rng(3)
    n = 40
    seq = np.repeat(np.arange(2, dtype=np.int32), n // 2)
    pos = np.concatenate([rng.choice(int(inp.seq_lens[b]), n // 2, replace=False)
                          for b in range(2)]).astype(np.int32)
    rope_pos = rng.integers(0, 1 << 20, n).astype(np.int32)
    c = workload.round_bf16((rng.standard_normal((n, wl.kv_rank)) *
                             rng.uniform(0.05, 20, (n, 1))).astype(np.float32))
    k = workload.round_bf16(rng.standard_normal((n, wl.rope_dim)).astype(np.float32))
    c[0] = c[0, 0]                                   # a constant latent part: step 0
    pool = torch.full((inp.num_pages, wl.page_size, wl.dim + 16), 255, dtype=torch.uint8,
                      device="cuda")
    mla.cache_append_q8(cfg, upload(c, torch.bfloat16), upload(k, torch.bfloat16),
                        upload(seq, torch.int32), upload(pos, torch.int32),
                        upload(rope_pos, torch.int32), upload(inp.page_table, torch.int32), pool,
                        mode)
    torch.cuda.synchronize()
    got = _pool_rows(pool, inp, wl, seq, pos)
    meta = got[:, wl.dim:].copy().view(np.float32)          # [n][4]
    krot = (oracle.rotated_keys_f32(k, rope_pos, wl.rope_base) if mode == mla.APPEND_ROTATE
            else k)
    rows, c_hat, k_hat = oracle.quantize_cache_rows(c, krot)
    dc = wl.kv_rank
    # latent part: the inputs are the same bf16 values on both sides -> bit-exact
    assert np.array_equal(got[:, :dc], rows["codes"][:, :dc])
    assert np.array_equal(meta[:, 0], rows["lat_min"]) and np.array_equal(meta[:, 1],
                                                                            rows["lat_step"])
    assert meta[0, 1] == 0 and np.all(got[0, :dc] == 0)
    if mode == mla.APPEND_RAW:  # RoPE part coded as given -> bit-exact too
        assert np.array_equal(got[:, dc:wl.dim], rows["codes"][:, dc:])
        assert np.array_equal(meta[:, 2], rows["rope_min"])
        assert np.array_equal(meta[:, 3], rows["rope_step"])
    else:
        # rotated in fp64 on both sides by different sin/cos routines: the
        # float32 keys may differ in their last bit, so a code may move by one
        dcode = np.abs(got[:, dc:wl.dim].astype(int) - rows["codes"][:, dc:].astype(int))
        assert dcode.max() <= 1 and (dcode > 0).mean() < 1e-2
        np.testing.assert_allclose(meta[:, 2], rows["rope_min"], rtol=1e-6)
        np.testing.assert_allclose(meta[:, 3], rows["rope_step"], rtol=1e-5)


def test_q8_invalid_sequence_gives_nan_only_there():
    wl = small("v2lite_paged_varlen", batch=3, len_range=(100, 500), num_splits=2, cache="q8")
    inp = workload.make(wl, 5)
    case = Case(wl, inputs=inp)
    bad_lens = inp.seq_lens.copy()
    bad_lens[1] = wl.max_seq_len + 64            # beyond max_seq_len: invalid
    st = case.step
    st.absorb(case.q_nope, case.q_rope, case.w_uk)
    st.decode(case.pool, case.pt, upload(bad_lens, torch.int32))
    st.combine()
    st.up_project(case.w_uv)
    torch.cuda.synchronize()
    got = case.results()
    assert np.all(np.isnan(got["lse"][1])) and np.all(np.isnan(got["o"][1]))
    check_against_oracle(case, got, case.oracle(seqs=[0, 2]), seqs=[0, 2])


# ---------------------------------------------------------------- row scales
# The decode feeds fp16 MFMA operands: the query parts and P = p * step. Each
# is scaled by a power of two per row inside the kernel, so the rows' own
# scales must not matter. Latents scaled by alpha with the content query
# scaled by 1/alpha (and the RoPE parts by beta, 1/beta) keep the scores and
# the softmax of the unit-scale workload while the steps and the query values
# move across 2^-16 .. 2^16 (powers of two: every value stays bf16-exact).
SCALED = small("v2lite_32k_q8", batch=2, seq_len=700, num_splits=3)


def _scaled_case(alpha, beta, seed=6):
    inp = workload.make(SCALED, seed)
    inp.c *= np.float32(alpha)
    inp.q_nope *= np.float32(1.0 / alpha)
    inp.k_rope *= np.float32(beta)
    inp.q_rope *= np.float32(1.0 / beta)
    return Case(SCALED, inputs=inp)


@pytest.mark.parametrize("alpha,beta", [(2.0 ** -14, 2.0 ** -14), (2.0 ** 14, 2.0 ** 14),
                                        (2.0 ** -16, 2.0 ** 16), (2.0 ** 7, 2.0 ** -7),
                                        (2.0 ** 22, 2.0 ** -20)],
                         ids=["2^-14", "2^14", "lat2^-16_rope2^16", "lat2^7_rope2^-7",
                              "lat2^22_rope2^-20"])
def test_q8_decode_scaled_rows(alpha, beta):
    case = _scaled_case(alpha, beta)
    case.run()
    check_against_oracle(case, case.results(), case.oracle())


def test_q8_decode_per_token_scales():
    # every cached row scaled by its own 2^u, u in [-14, 14] (latent and RoPE
    # parts separately): the steps of one sequence span 2^28, and the row a
    # query weights most is rarely the one with the largest step
    inp = workload.make(SCALED, 7)
    rng = np.random.default_rng(11)
    T = inp.c.shape[0]
    inp.c *= np.exp2(rng.integers(-14, 15, (T, 1))).astype(np.float32)
    inp.k_rope *= np.exp2(rng.integers(-14, 15, (T, 1))).astype(np.float32)
    inp.q_nope *= np.float32(2.0 ** -12)
    inp.q_rope *= np.float32(2.0 ** -12)
    case = Case(SCALED, inputs=inp)
    case.run()
    check_against_oracle(case, case.results(), case.oracle())


def test_q8_decode_constant_and_narrow_parts():
    # a tenth of the rows with a constant latent part (step 0), a tenth with a
    # zero RoPE key (a constant rotated part), a tenth with a latent part
    # 3 + 2^-6 N(0, 1) (a few levels of a narrow range far from zero)
    inp = workload.make(SCALED, 8)
    rng = np.random.default_rng(12)
    T = inp.c.shape[0]
    kind = rng.integers(0, 10, T)
    const = kind == 0
    inp.c[const] = workload.round_bf16(rng.standard_normal((int(const.sum()), 1))
                                       .astype(np.float32)) * np.ones((1, SCALED.kv_rank),
                                                                      np.float32)
    inp.k_rope[kind == 1] = 0.0
    narrow = kind == 2
    inp.c[narrow] = workload.round_bf16(
        (3.0 + rng.standard_normal((int(narrow.sum()), SCALED.kv_rank)) / 64.0).astype(np.float32))
    # the newest row of each sequence (the one every step re-appends) constant
    for b in range(SCALED.batch):
        inp.c[int(inp.offsets[b + 1]) - 1] = np.float32(-0.75)
    case = Case(SCALED, inputs=inp)
    case.run()
    check_against_oracle(case, case.results(), case.oracle())
