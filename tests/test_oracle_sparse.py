"""Pins of the oracle's sparse read against what fixes it independently.

The sparse read ("DeepSeek's Config Says 16 KV Heads, Its Cache Holds a Ninth
of That", section 6, "Sparse attention"): a small scorer rates every cached
token for each query and attention reads only the top-k of them; the cache
itself keeps every token. The pins: a scalar-loop brute force of the scores
and of attention over a selection, closed forms (one-hot head weights give one
head's ReLU dot; a single selected token gives its own latent), additivity in
the head weights, the selection's order properties on tied scores, dense
attention when k covers the sequence, and planted mistakes that the battery
must catch.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute, mla_ref
import workload


def _idx_case(seed, Q=2, Hi=3, di=5, L=9):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Q, Hi, di)), rng.standard_normal((Q, Hi)),
            rng.standard_normal((L, di)))


def _attn_case(seed, H=2, dn=4, dv=4, dc=8, dr=4, L=11, Q=2):
    rng = np.random.default_rng(seed)
    return dict(c=rng.standard_normal((L, dc)), kr=rng.standard_normal((L, dr)),
                qn=rng.standard_normal((Q, H, dn)), qr=rng.standard_normal((Q, H, dr)),
                w_uk=rng.standard_normal((H, dn, dc)) / math.sqrt(dc),
                w_uv=rng.standard_normal((H, dv, dc)) / math.sqrt(dc),
                scale=1.0 / math.sqrt(dn + dr))


def _sparse(k, sel):
    L, Q = len(k["c"]), len(k["qn"])
    keep = np.zeros((Q, L), dtype=bool)
    for j in range(Q):
        keep[j, sel[j]] = True
    return oracle.attend_sequence(k["c"], k["kr"], k["qn"], k["qr"], k["w_uk"], k["w_uv"],
                                  k["scale"], keep=keep)


# ---------------------------------------------------------------- index scores
def _scores_brute_ok(seed):
    q, w, kk = _idx_case(seed)
    got = oracle.indexer_scores(q, w, kk)
    ref = np.array(brute.brute_index_scores(q.tolist(), w.tolist(), kk.tolist()))
    return bool(np.allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max())))


def _scores_closed_forms_ok(seed):
    q, w, kk = _idx_case(seed, Hi=4)
    ok = True
    for h in range(4):  # one-hot weights: one head's ReLU dot
        oh = np.zeros_like(w)
        oh[:, h] = 1.0
        want = np.maximum(np.einsum("qd,td->qt", q[:, h], kk), 0.0)
        ok &= np.allclose(oracle.indexer_scores(q, oh, kk), want, rtol=0, atol=1e-12)
    # additive in the head weights, negative weights included
    w2 = -np.abs(w) * 0.7
    lhs = oracle.indexer_scores(q, w + w2, kk)
    rhs = oracle.indexer_scores(q, w, kk) + oracle.indexer_scores(q, w2, kk)
    ok &= np.allclose(lhs, rhs, rtol=0, atol=1e-12)
    # a key opposite to every query head scores 0
    neg = -np.abs(q[0, 0])[None, :] * np.sign(q[0, 0])[None, :]
    ok &= np.allclose(oracle.indexer_scores(q[:1, :1], w[:1, :1], neg), 0.0)
    return bool(ok)


@pytest.mark.parametrize("seed", range(4))
def test_index_scores_brute_force(seed):
    assert _scores_brute_ok(seed)


def test_index_scores_closed_forms():
    for seed in range(3):
        assert _scores_closed_forms_ok(seed)


# ---------------------------------------------------------------- top-k
def test_topk_hand_examples():
    s = [0.5, 2.0, -1.0, 2.0, 7.0, 2.0, 0.0]
    assert oracle.topk_tokens(s, 1, 7).tolist() == [4]
    assert oracle.topk_tokens(s, 2, 7).tolist() == [1, 4]         # ties: smaller index
    assert oracle.topk_tokens(s, 3, 7).tolist() == [1, 3, 4]
    assert oracle.topk_tokens(s, 4, 7).tolist() == [1, 3, 4, 5]
    assert oracle.topk_tokens(s, 3, 4).tolist() == [0, 1, 3]      # only 0..3 visible
    assert oracle.topk_tokens(s, 9, 5).tolist() == [0, 1, 2, 3, 4]  # k covers them
    assert oracle.topk_tokens([0.0, -0.0, 0.0], 2, 3).tolist() == [0, 1]  # -0 == +0
    assert oracle.topk_tokens([-np.inf, 1.0, -np.inf], 2, 3).tolist() == [0, 1]
    with pytest.raises(ValueError):
        oracle.topk_tokens([1.0, np.nan, 0.0], 1, 3)


def _topk_ok(s, k, visible):
    sel = oracle.topk_tokens(s, k, visible)
    s = np.asarray(s, np.float64)[:visible]
    n = min(k, visible)
    if len(sel) != n or len(set(sel.tolist())) != n or not np.all(np.diff(sel) > 0):
        return False
    if not (np.all(sel >= 0) and np.all(sel < visible)):
        return False
    rest = np.setdiff1d(np.arange(visible), sel)
    if len(rest) == 0:
        return True
    lo, hi = s[sel].min(), s[rest].max()
    if lo < hi:
        return False
    if lo == hi:  # the boundary value: selected copies precede the others
        return bool(sel[s[sel] == lo].max() < rest[s[rest] == lo].min())
    return True


@pytest.mark.parametrize("length,k", [(40, 7), (300, 64), (1000, 999), (1000, 1), (64, 64)])
def test_topk_order_properties_with_ties(length, k):
    rows = workload.score_rows(3, 4, length)
    for r in rows:
        for visible in (length, length - 1, max(1, length // 2)):
            assert _topk_ok(r, k, visible)


# ---------------------------------------------------------------- attention over a selection
def _sparse_brute_ok(seed):
    k = _attn_case(seed)
    L, Q = len(k["c"]), len(k["qn"])
    rng = np.random.default_rng(seed + 50)
    sel = [np.sort(rng.choice(L - Q + j + 1, size=4, replace=False)) for j in range(Q)]
    o, ol, lse = _sparse(k, sel)
    bo, bol, blse = brute.brute_sequence(k["c"].tolist(), k["kr"].tolist(), k["qn"].tolist(),
                                         k["qr"].tolist(), k["w_uk"].tolist(),
                                         k["w_uv"].tolist(), k["scale"],
                                         selected=[s.tolist() for s in sel])
    return bool(np.allclose(o, bo, rtol=0, atol=1e-12 * np.abs(bo).max())
                and np.allclose(ol, bol, rtol=0, atol=1e-12 * np.abs(bol).max())
                and np.allclose(lse, blse, rtol=1e-12, atol=0))


@pytest.mark.parametrize("seed", range(4))
def test_sparse_attention_brute_force(seed):
    assert _sparse_brute_ok(seed)


def test_single_selected_token_gives_its_own_rows():
    k = _attn_case(5)
    L, Q = len(k["c"]), len(k["qn"])
    t = 3
    o, ol, lse = _sparse(k, [[t]] * Q)
    for j in range(Q):
        for h in range(len(k["w_uk"])):
            np.testing.assert_allclose(ol[j, h], k["c"][t], rtol=0, atol=1e-14)
            np.testing.assert_allclose(o[j, h], k["w_uv"][h] @ k["c"][t], rtol=0, atol=1e-14)


def test_selecting_an_invisible_token_is_refused():
    k = _attn_case(6)
    L, Q = len(k["c"]), len(k["qn"])
    with pytest.raises(ValueError):
        _sparse(k, [[L - Q + 1], [0]])  # query 0 sits at L - Q


def test_topk_covering_the_sequence_is_dense_attention():
    wl = workload.WORKLOADS["tiny_f32"].replace(batch=2, q_len=3, seq_len=70, index_topk=70,
                                                index_heads=4, index_dim=8)
    inp = workload.make(wl, 4)
    dense = oracle.mla_decode_ref(inp)
    sp = oracle.mla_decode_ref_sparse(inp)
    for key in ("o", "o_lat", "lse"):
        np.testing.assert_array_equal(sp[key], dense[key])
    for b in range(2):
        for j in range(3):
            assert sp["selection"][b][j].tolist() == list(range(70 - 3 + j + 1))


def test_workload_selection_is_seeded_and_sized():
    wl = workload.WORKLOADS["tiny_f32"].replace(batch=2, q_len=2, seq_len=300, index_topk=50,
                                                index_heads=4, index_dim=8)
    inp = workload.make(wl, 9)
    a, b = oracle.dsa_selection(inp), oracle.dsa_selection(workload.make(wl, 9))
    for x, y in zip(a, b):
        for u, v in zip(x, y):
            assert u.tolist() == v.tolist() and len(u) == 50 and u.max() < 300


# ---------------------------------------------------------------- planted mistakes
def _battery():
    ok = True
    for seed in (400, 401):
        ok &= _scores_brute_ok(seed) and _scores_closed_forms_ok(seed)
        ok &= _sparse_brute_ok(seed)
    for r in workload.score_rows(8, 3, 200):
        ok &= _topk_ok(r, 30, 200) and _topk_ok(r, 30, 150)
    return bool(ok)


def _idx_no_relu(q_idx, w_idx, k_idx):
    q, w, k = (np.asarray(x, np.float64) for x in (q_idx, w_idx, k_idx))
    return np.einsum("qh,qht->qt", w, np.matmul(q, k.T))


def _idx_relu_after_weight(q_idx, w_idx, k_idx):
    q, w, k = (np.asarray(x, np.float64) for x in (q_idx, w_idx, k_idx))
    return np.maximum(np.einsum("qh,qht->qt", w, np.matmul(q, k.T)), 0.0)


def _topk_smallest(scores, k, visible):
    s = np.asarray(scores, np.float64)[:visible]
    if visible <= k:
        return np.arange(visible)
    return np.sort(np.lexsort((np.arange(visible), s))[:k])


def _topk_ties_high(scores, k, visible):
    s = np.asarray(scores, np.float64)[:visible]
    if visible <= k:
        return np.arange(visible)
    return np.sort(np.lexsort((-np.arange(visible), -s))[:k])


def _topk_sees_one_more(scores, k, visible):
    return mla_ref._orig_topk(scores, k, min(visible + 1, len(scores)))


def _attend_ignores_keep(*args, keep=None, **kw):
    return mla_ref._orig_attend(*args, **kw)


@pytest.mark.parametrize("target,mutant", [
    ("indexer_scores", _idx_no_relu),
    ("indexer_scores", _idx_relu_after_weight),
    ("topk_tokens", _topk_smallest),
    ("topk_tokens", _topk_ties_high),
    ("topk_tokens", _topk_sees_one_more),
    ("attend_sequence", _attend_ignores_keep),
])
def test_planted_sparse_mistakes_are_caught(monkeypatch, target, mutant):
    assert _battery(), "clean oracle must pass the battery"
    monkeypatch.setattr(mla_ref, "_orig_topk", mla_ref.topk_tokens, raising=False)
    monkeypatch.setattr(mla_ref, "_orig_attend", mla_ref.attend_sequence, raising=False)
    monkeypatch.setattr(mla_ref, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    assert not _battery(), f"planted mistake in {target} went unnoticed"
