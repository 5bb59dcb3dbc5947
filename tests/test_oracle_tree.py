"""Pins of the oracle's tree verification against what fixes it independently.

Tree verification ("The Architecture of Memory", "Tree Attention
Verification"): the prefix is seen by every drafted query with no mask; among
the drafted tokens a query sees only its own branch, so independent branches
never attend to one another; and verification must give what decoding the
branch token by token would ("Speculative Decoding: Amortizing the Memory
Fetch"). The pins: a chain-shaped tree is the chain, every branch equals
sequential single-token decode of prefix + branch (positions included), a
pure-Python brute force on tiny inputs, absorbed == unabsorbed, split + LSE
merge, independence from other branches, and planted mistakes that each pin
battery must catch.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute, mla_ref
import workload


def _case(seed, H=2, dn=8, dv=8, dc=16, dr=8, L=37, Q=6, parents=None):
    rng = np.random.default_rng(seed)
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    c, kr = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    qn, qr = rng.standard_normal((Q, H, dn)), rng.standard_normal((Q, H, dr))
    if parents is None:
        parents = [-1] + [int(rng.integers(-1, j)) for j in range(1, Q)]
    return dict(w_uk=w_uk, w_uv=w_uv, c=c, kr=kr, qn=qn, qr=qr, parents=list(parents),
                scale=1.0 / math.sqrt(dn + dr))


def _tree(k, **kw):
    return oracle.attend_sequence(k["c"], k["kr"], k["qn"], k["qr"], k["w_uk"], k["w_uv"],
                                  k["scale"], chunk=7, parents=k["parents"], **kw)


def _branch(parents, j):
    """Drafted tokens from the prefix down to j (root first)."""
    path = []
    while j != -1:
        path.append(j)
        j = parents[j]
    return path[::-1]


def _sequential_ok(k, tol=1e-12):
    o, ol, lse = _tree(k)
    L, Q = len(k["c"]), len(k["parents"])
    pre = L - Q
    ok = True
    for j in range(Q):
        rows = list(range(pre)) + [pre + i for i in _branch(k["parents"], j)]
        oj, olj, lj = oracle.attend_sequence(k["c"][rows], k["kr"][rows], k["qn"][j:j + 1],
                                             k["qr"][j:j + 1], k["w_uk"], k["w_uv"], k["scale"])
        ok &= np.allclose(o[j], oj[0], rtol=0, atol=tol * np.abs(oj).max())
        ok &= np.allclose(ol[j], olj[0], rtol=0, atol=tol * np.abs(olj).max())
        ok &= np.allclose(lse[j], lj[0], rtol=tol, atol=0)
    return bool(ok)


def _brute_ok(k, tol=1e-12):
    o, ol, lse = _tree(k)
    bo, bol, blse = brute.brute_sequence(k["c"].tolist(), k["kr"].tolist(), k["qn"].tolist(),
                                         k["qr"].tolist(), k["w_uk"].tolist(), k["w_uv"].tolist(),
                                         k["scale"], parents=k["parents"])
    return bool(np.allclose(o, bo, rtol=0, atol=tol * np.abs(bo).max())
                and np.allclose(ol, bol, rtol=0, atol=tol * np.abs(bol).max())
                and np.allclose(lse, blse, rtol=tol, atol=0))


# ---------------------------------------------------------------- structure
def test_depths_ancestry_positions_closed_forms():
    par = [-1, 0, 0, 1, -1, 4, 3]
    assert oracle.tree_depths(par).tolist() == [0, 1, 1, 2, 0, 1, 3]
    anc = oracle.tree_ancestry(par)
    assert np.flatnonzero(anc[6]).tolist() == [0, 1, 3, 6]
    assert np.flatnonzero(anc[5]).tolist() == [4, 5]
    assert np.flatnonzero(anc[2]).tolist() == [0, 2]
    kp, qp = oracle.tree_positions(20, par)
    assert kp[:13].tolist() == list(range(13))
    assert kp[13:].tolist() == [13, 14, 14, 15, 13, 14, 16] == qp.tolist()
    ex = oracle.tree_excluded(20, par)
    assert not ex[:, :13].any()                       # the prefix is never masked
    assert ex[2, 13 + 1] and not ex[2, 13 + 0]        # sibling hidden, parent seen
    for bad in ([0], [-1, 1], [-1, 0, 3], [-2]):
        with pytest.raises(ValueError):
            oracle.tree_depths(bad)


def test_chain_shaped_tree_is_the_chain():
    for seed in range(3):
        k = _case(seed, parents=[-1, 0, 1, 2, 3, 4])
        o, ol, lse = _tree(k)
        co, col, clse = oracle.attend_sequence(k["c"], k["kr"], k["qn"], k["qr"], k["w_uk"],
                                               k["w_uv"], k["scale"], chunk=7)
        assert np.array_equal(o, co) and np.array_equal(ol, col) and np.array_equal(lse, clse)


# ---------------------------------------------------------------- sequential equivalence
@pytest.mark.parametrize("seed", range(6))
def test_every_branch_equals_sequential_decode(seed):
    assert _sequential_ok(_case(100 + seed))


def test_all_roots_each_draft_sees_prefix_and_itself():
    k = _case(7, Q=5, parents=[-1] * 5)
    assert _sequential_ok(k)
    o, ol, lse = _tree(k)
    L, Q = len(k["c"]), 5
    for j in range(Q):  # position L - Q for every draft
        rows = list(range(L - Q)) + [L - Q + j]
        oj, _, lj = oracle.attend_sequence(k["c"][rows], k["kr"][rows], k["qn"][j:j + 1],
                                           k["qr"][j:j + 1], k["w_uk"], k["w_uv"], k["scale"])
        np.testing.assert_allclose(o[j], oj[0], rtol=0, atol=1e-13 * np.abs(oj).max())


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(4))
def test_tree_brute_force_agrees(seed):
    assert _brute_ok(_case(200 + seed, H=2, dn=4, dv=4, dc=8, dr=4, L=9, Q=5))


# ---------------------------------------------------------------- algebra
def test_tree_absorbed_equals_unabsorbed():
    k = _case(11, Q=7)
    o, ol, lse = _tree(k)
    ao, aol, alse = oracle.absorbed_attend_sequence(k["c"], k["kr"], k["qn"], k["qr"], k["w_uk"],
                                                    k["w_uv"], k["scale"], parents=k["parents"])
    np.testing.assert_allclose(o, ao, rtol=0, atol=1e-12 * np.abs(o).max())
    np.testing.assert_allclose(ol, aol, rtol=0, atol=1e-12 * np.abs(ol).max())
    np.testing.assert_allclose(lse, alse, rtol=1e-12)


@pytest.mark.parametrize("S,chunk", [(1, 0), (3, 0), (5, 0), (4, 32)])
def test_tree_split_merge_equals_unsplit(S, chunk):
    k = _case(12, L=70, Q=8)
    _, ol, lse = _tree(k)
    op, lp = oracle.attend_partials(k["c"], k["kr"], k["qn"], k["qr"], k["w_uk"], k["scale"], S,
                                    page=16, chunk_tokens=chunk, parents=k["parents"])
    mo, ml = oracle.lse_combine(op, lp)
    np.testing.assert_allclose(mo, ol, rtol=0, atol=1e-12 * np.abs(ol).max())
    np.testing.assert_allclose(ml, lse, rtol=1e-13)


def test_other_branches_do_not_reach_a_query():
    k = _case(13, Q=7, parents=[-1, 0, 0, 1, 2, -1, 5])
    o, ol, lse = _tree(k)
    L, Q = len(k["c"]), 7
    pre = L - Q
    for j in range(Q):
        off = [i for i in range(Q) if i not in _branch(k["parents"], j)]
        k2 = dict(k, c=k["c"].copy(), kr=k["kr"].copy())
        k2["c"][[pre + i for i in off]] += 5.0
        k2["kr"][[pre + i for i in off]] -= 3.0
        o2, ol2, lse2 = _tree(k2)
        assert np.array_equal(o2[j], o[j]) and np.array_equal(lse2[j], lse[j])
        # ... while changing the query's own parent (if any) does
        if k["parents"][j] >= 0:
            k3 = dict(k, c=k["c"].copy())
            k3["c"][pre + k["parents"][j]] += 1.0
            assert not np.allclose(_tree(k3)[0][j], o[j])


def test_workload_trees_are_valid_and_seeded():
    wl = workload.WORKLOADS["tiny_f32"].replace(batch=4, q_len=9, tree="random")
    p0 = workload.make(wl, 3, with_latents=False).parents
    p1 = workload.make(wl, 3, with_latents=False).parents
    assert np.array_equal(p0, p1)
    for row in p0:
        oracle.tree_depths(row)  # raises on an invalid order
    assert workload.make(wl.replace(tree=None), 3, with_latents=False).parents is None


# ---------------------------------------------------------------- planted mistakes
def _battery():
    ok = True
    for seed in (300, 301):
        ok &= _sequential_ok(_case(seed))
        ok &= _brute_ok(_case(seed, H=2, dn=4, dv=4, dc=8, dr=4, L=9, Q=5))
    return bool(ok)


def _mut_slot_positions(seq_len, parents):
    Q = len(parents)
    return np.arange(seq_len), seq_len - Q + np.arange(Q)


def _mut_depth_from_one(seq_len, parents):
    kp, qp = mla_ref._orig_positions(seq_len, parents)
    pre = seq_len - len(parents)
    kp = kp.copy()
    kp[pre:] += 1
    return kp, qp + 1


def _mut_query_only_positions(seq_len, parents):
    kp, qp = mla_ref._orig_positions(seq_len, parents)
    return np.arange(seq_len), qp


def _mut_siblings_visible(seq_len, parents):
    return np.zeros((len(parents), seq_len), dtype=bool)


def _mut_self_hidden(seq_len, parents):
    ex = mla_ref._orig_excluded(seq_len, parents)
    pre = seq_len - len(parents)
    for j in range(len(parents)):
        ex[j, pre + j] = True
    return ex


@pytest.mark.parametrize("target,mutant", [
    ("tree_positions", _mut_slot_positions),
    ("tree_positions", _mut_depth_from_one),
    ("tree_positions", _mut_query_only_positions),
    ("tree_excluded", _mut_siblings_visible),
    ("tree_excluded", _mut_self_hidden),
])
def test_planted_tree_mistakes_are_caught(monkeypatch, target, mutant):
    assert _battery(), "clean oracle must pass the battery"
    monkeypatch.setattr(mla_ref, "_orig_positions", mla_ref.tree_positions, raising=False)
    monkeypatch.setattr(mla_ref, "_orig_excluded", mla_ref.tree_excluded, raising=False)
    monkeypatch.setattr(mla_ref, target, mutant)
    assert not _battery(), f"planted mistake in {target} went unnoticed"
