"""GPU check of the no-allocation top-k entry point, through the C ABI.

mla_index_scores_topk_noalloc keeps the top-k workspace in a device array
inside the library instead of a caller buffer; it must give what
mla_index_scores_topk gives with a caller workspace (the same kernels):
scores, indices and counts bit for bit. Two calls in a row, the second on a
smaller input, so whatever the first left in the library's array is what the
second starts from; plus a shape that takes the generic (non-MFMA) indexer
and one with invalid sequences, whose rows the selection must still clear.
"""
import numpy as np
import pytest
import torch

import workload
import mla_latent_kv_03_amd as mla
from mla_latent_kv_03_amd.pipeline import upload

from gpu_case import Case

pytestmark = pytest.mark.gpu

W = workload.WORKLOADS


def _both(case, seq_lens=None):
    """(scores, indices, counts) from the caller-workspace call and from the
    no-alloc call, on fresh output buffers with different fill values."""
    st = case.step
    q_idx, w_idx, _, ipool = case.sparse
    lens = case.seq_lens if seq_lens is None else seq_lens
    B, Q, K = st.batch, st.q_len, st.index_topk
    outs = []
    for noalloc in (False, True):
        fill = 5 if noalloc else -5
        scores = torch.full_like(st.scores, float(fill))
        idx = torch.full((B, Q, K), fill, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, Q), fill, dtype=torch.int32, device="cuda")
        if noalloc:
            mla.index_scores_topk_noalloc(case.cfg, q_idx, w_idx, ipool, case.pt, lens, scores,
                                          st.max_seq_len, idx, cnt)
        else:
            mla.index_scores_topk(case.cfg, q_idx, w_idx, ipool, case.pt, lens, scores,
                                  st.max_seq_len, idx, cnt, st.topk_ws)
        torch.cuda.synchronize()
        outs.append((scores.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()))
    return outs


def _same(a, b, lens, Q):
    sa, ia, ca = a
    sb, ib, cb = b
    assert np.array_equal(ca, cb)
    for bb, L in enumerate(lens):
        # scores of the cached tokens (entries past L_b are not written)
        assert np.array_equal(sa[bb, :, :L].view(np.uint32), sb[bb, :, :L].view(np.uint32))
        for j in range(Q):
            n = int(ca[bb, j])
            if n > 0:
                assert np.array_equal(ia[bb, j, :n], ib[bb, j, :n]), (bb, j)


def test_noalloc_topk_matches_caller_workspace_twice():
    big = W["v2lite_32k_dsa"].replace(batch=3, q_len=2, seq_len=None, len_range=(2500, 6000),
                                      paged=True, index_topk=512, num_splits=4)
    small = big.replace(batch=2, q_len=1, len_range=(700, 1500), index_topk=256)
    for wl, seed in ((big, 1), (small, 2)):
        print(f"[gpu] noalloc top-k {wl.batch}x{wl.q_len} topk {wl.index_topk} seed {seed}",
              flush=True)
        case = Case(wl, seed=seed)
        a, b = _both(case)
        _same(a, b, [int(x) for x in case.inp.seq_lens], wl.q_len)
        assert np.all(a[2] >= 0)


def test_noalloc_topk_generic_indexer_and_invalid_sequences():
    wl = W["v2lite_32k_dsa"].replace(batch=3, q_len=2, seq_len=None, len_range=(300, 900),
                                     paged=True, index_topk=100, index_heads=8, index_dim=64,
                                     num_splits=2)
    case = Case(wl, seed=3)
    bad = case.inp.seq_lens.copy()
    bad[1] = wl.max_seq_len + 5                 # beyond max_seq_len: count -1
    lens = upload(bad, torch.int32)
    a, b = _both(case, lens)
    assert np.all(a[2][1] == -1) and np.array_equal(a[2], b[2])
    good = [int(bad[0]), 0, int(bad[2])]        # sequence 1's scores are not written
    _same(a, b, good, wl.q_len)
    # a valid call after the invalid one: the array was left clear
    a, b = _both(case)
    _same(a, b, [int(x) for x in case.inp.seq_lens], wl.q_len)


def test_noalloc_topk_rejects_more_queries_than_it_holds():
    wl = W["v2lite_32k_dsa"].replace(batch=mla.TOPK_NOALLOC_MAX_QUERIES + 1, q_len=1,
                                     seq_len=64, index_topk=16, num_splits=1)
    cfg = mla.Config.from_workload(wl)
    B = wl.batch
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(shape, dtype=dt, device="cuda")  # noqa
    with pytest.raises(mla.MLAError) as e:
        mla.index_scores_topk_noalloc(cfg, z(B, 1, 64, 128), z(B, 1, 64, dt=torch.float32),
                                      z(B, 64, 128), z(B, 1, dt=torch.int32),
                                      z(B, dt=torch.int32), z(B, 1, 64, dt=torch.float32), 64,
                                      z(B, 1, 16, dt=torch.int32), z(B, dt=torch.int32))
    assert e.value.status == 5  # MLA_ERR_CAPACITY, before any launch
