"""Pins of the oracle's 8-bit latent cache against what fixes it independently.

The cache quantization ("KV Cache Optimization: Scaling to Million-Token
Contexts", technique 3 and its comparison table): each row part is coded in 8
bits between its own minimum and maximum. The pins are properties a wrong
quantizer breaks (reconstruction within half a step, the extremes at codes 0
and 255, monotone codes, constant parts), a lossless case where quantized and
unquantized attention must agree exactly, the rotated-key entry point against
the main oracle, and planted mistakes that the battery must catch.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import mla_ref
import workload


def _rows(seed, n=20, d=512):
    rng = np.random.default_rng(seed)
    out = [rng.standard_normal(d).astype(np.float32)]
    out.append((rng.standard_normal(d) * 40 + 7).astype(np.float32))            # wide, offset
    out.append(rng.uniform(-1e-3, 1e-3, d).astype(np.float32))                  # narrow
    out.append(np.where(rng.random(d) < 0.02, 30.0, rng.standard_normal(d)).astype(np.float32))
    out.extend((rng.standard_normal((n, d)) * rng.uniform(0.1, 5, (n, 1))).astype(np.float32))
    return out


def _quantizer_ok(x):
    q, mn, step = oracle.quantize_q8(x)
    x = np.asarray(x, np.float64)
    if step == 0:
        return bool(np.all(q == 0) and np.all(oracle.dequantize_q8(q, mn, step) == x))
    deq = oracle.dequantize_q8(q, mn, step)
    ok = np.max(np.abs(deq - x)) <= step * (0.5 + 1e-4)          # within half a step
    ok &= q[np.argmin(x)] == 0 and q[np.argmax(x)] == oracle.Q8_LEVELS  # extremes
    order = np.argsort(x, kind="stable")
    ok &= bool(np.all(np.diff(q[order].astype(int)) >= 0))      # monotone
    ok &= abs(float(mn) - x.min()) == 0.0                       # the range starts at the min
    ok &= abs(float(mn) + oracle.Q8_LEVELS * float(step) - x.max()) <= 1e-5 * max(1.0, abs(x.max()))
    return bool(ok)


@pytest.mark.parametrize("seed", range(3))
def test_quantizer_properties(seed):
    for x in _rows(seed):
        assert _quantizer_ok(x)


def test_quantizer_closed_forms():
    x = np.arange(256, dtype=np.float32)                   # step exactly 1
    q, mn, step = oracle.quantize_q8(x)
    assert mn == 0 and step == 1 and np.array_equal(q, np.arange(256))
    q, mn, step = oracle.quantize_q8(np.array([-1.0, 1.0, 0.0], np.float32))
    assert q[0] == 0 and q[1] == 255 and mn == -1 and step == np.float32(2 / 255)
    assert q[2] in (127, 128)                               # the midpoint
    q, mn, step = oracle.quantize_q8(np.full(9, 2.5, np.float32))
    assert step == 0 and np.all(q == 0) and np.all(oracle.dequantize_q8(q, mn, step) == 2.5)


def _lossless_case(seed, L=40, Q=3, H=2, dn=8, dv=8, dc=32, dr=8):
    """Rows whose parts are exactly mn + code * step with codes 0 and 255
    present and power-of-two steps: 8-bit coding loses nothing on them."""
    rng = np.random.default_rng(seed)

    def exact_part(n):
        codes = rng.integers(0, 256, n)
        codes[rng.integers(0, n)] = 0
        codes[(rng.integers(0, n - 1) + 1 + np.argmin(codes)) % n] = 255
        step = 2.0 ** -int(rng.integers(4, 9))
        mn = step * int(rng.integers(-300, 300))
        return (mn + codes * step).astype(np.float32)

    c = np.stack([exact_part(dc) for _ in range(L)])
    kr = np.stack([exact_part(dr) for _ in range(L)])        # taken as the rotated keys
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    qn, qr = rng.standard_normal((Q, H, dn)), rng.standard_normal((Q, H, dr))
    return c, kr, qn, qr, w_uk, w_uv, 1.0 / math.sqrt(dn + dr)


def test_lossless_rows_give_the_unquantized_attention():
    for seed in range(3):
        c, kr, qn, qr, w_uk, w_uv, sc = _lossless_case(seed)
        rows, c_hat, k_hat = oracle.quantize_cache_rows(c, kr)
        assert np.array_equal(c_hat, c.astype(np.float64))
        assert np.array_equal(k_hat, kr.astype(np.float64))
        o, ol, lse = oracle.attend_sequence_rotated(c_hat, k_hat, qn, qr, w_uk, w_uv, sc)
        o2, ol2, lse2 = oracle.attend_sequence_rotated(c, kr, qn, qr, w_uk, w_uv, sc)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_rotated_key_entry_equals_main_oracle():
    wl = workload.WORKLOADS["tiny_f32"].replace(q_len=3, seq_len=70)
    inp = workload.make(wl, 2)
    c, kr = inp.seq(0)
    o, ol, lse = oracle.attend_sequence(c, kr, inp.q_nope[0], inp.q_rope[0], inp.w_uk, inp.w_uv,
                                        wl.softmax_scale, wl.rope_base)
    k_rot = oracle.rope(kr, np.arange(70), wl.rope_base)
    o2, ol2, lse2 = oracle.attend_sequence_rotated(c, k_rot, inp.q_nope[0], inp.q_rope[0],
                                                   inp.w_uk, inp.w_uv, wl.softmax_scale,
                                                   wl.rope_base)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13 * np.abs(o).max())
    np.testing.assert_allclose(ol2, ol, rtol=0, atol=1e-13 * np.abs(ol).max())
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)
    # ... and with a drafted tree (keys rotated at prefix + depth)
    par = [-1, 0, -1]
    o, _, lse = oracle.attend_sequence(c, kr, inp.q_nope[0], inp.q_rope[0], inp.w_uk, inp.w_uv,
                                       wl.softmax_scale, wl.rope_base, parents=par)
    kp, _ = oracle.tree_positions(70, par)
    o2, _, lse2 = oracle.attend_sequence_rotated(c, oracle.rope(kr, kp, wl.rope_base),
                                                 inp.q_nope[0], inp.q_rope[0], inp.w_uk,
                                                 inp.w_uv, wl.softmax_scale, wl.rope_base,
                                                 parents=par)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13 * np.abs(o).max())


def test_q8_oracle_stays_near_the_unquantized_one():
    # the coding error shrinks the closer the 8-bit grid fits: the bf16-shaped
    # workload's q8 result lies within a few percent of the exact one
    wl = workload.WORKLOADS["v2lite_32k"].replace(batch=2, seq_len=300)
    inp = workload.make(wl, 1)
    ref = oracle.mla_decode_ref(inp)
    q8 = oracle.mla_decode_ref_q8(inp)
    for key in ("o", "o_lat"):
        err = np.abs(q8[key] - ref[key]).max() / np.abs(ref[key]).max()
        assert 0 < err < 3e-2, (key, err)
    assert np.abs(q8["lse"] - ref["lse"]).max() < 3e-2


# ---------------------------------------------------------------- planted mistakes
def _battery():
    ok = all(_quantizer_ok(x) for x in _rows(7, n=4))
    for seed in range(2):
        c, kr, qn, qr, w_uk, w_uv, sc = _lossless_case(seed)
        _, c_hat, k_hat = oracle.quantize_cache_rows(c, kr)
        ok &= np.array_equal(c_hat, c.astype(np.float64)) and np.array_equal(k_hat, kr)
    return bool(ok)


def _q_floor(x):
    x = np.asarray(x, np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(255))
    if step == 0:
        return np.zeros(x.shape, np.uint8), mn, step
    return np.clip(np.floor((x - mn) / step), 0, 255).astype(np.uint8), mn, step


def _q_256(x):
    x = np.asarray(x, np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(256))
    if step == 0:
        return np.zeros(x.shape, np.uint8), mn, step
    return np.clip(np.rint((x - mn) / step), 0, 255).astype(np.uint8), mn, step


def _q_from_max(x):
    x = np.asarray(x, np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(255))
    if step == 0:
        return np.zeros(x.shape, np.uint8), mn, step
    return np.clip(np.rint((mx - x) / step), 0, 255).astype(np.uint8), mn, step


def _rows_shared_range(c, k):
    rows, c_hat, k_hat = mla_ref._orig_rows(c, k)
    # the RoPE part coded on the latent part's range
    for t in range(len(k)):
        mn, st = rows["lat_min"][t], rows["lat_step"][t]
        q = np.clip(np.rint((np.asarray(k[t], np.float32) - mn) / st), 0, 255)
        k_hat[t] = oracle.dequantize_q8(q, mn, st)
    return rows, c_hat, k_hat


@pytest.mark.parametrize("target,mutant", [
    ("quantize_q8", _q_floor),
    ("quantize_q8", _q_256),
    ("quantize_q8", _q_from_max),
    ("quantize_cache_rows", _rows_shared_range),
])
def test_planted_q8_mistakes_are_caught(monkeypatch, target, mutant):
    assert _battery(), "clean oracle must pass the battery"
    monkeypatch.setattr(mla_ref, "_orig_rows", mla_ref.quantize_cache_rows, raising=False)
    monkeypatch.setattr(mla_ref, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    assert not _battery(), f"planted mistake in {target} went unnoticed"


# ---------------------------------------------------------------- drafted trees
# A drafted token of a tree is cached after its siblings but positioned one past
# its parent ("The Architecture of Memory", "Tree Attention Verification"), and
# verification must give what decoding its branch token by token would
# ("Speculative Decoding: Amortizing the Memory Fetch"). For the 8-bit cache
# that fixes where a drafted RoPE key is rotated before it is coded: at prefix
# + depth, where the chain of its branch would put it.
def _q8_tree_inputs(seed, L=45, Q=6, parents=None):
    wl = workload.WORKLOADS["tiny_f32"].replace(q_len=Q, seq_len=L, tree="random")
    inp = workload.make(wl, seed)
    if parents is not None:
        inp.parents = np.asarray([parents], np.int32)
    return inp


def _branch(parents, j):
    path = []
    while j != -1:
        path.append(j)
        j = int(parents[j])
    return path[::-1]


def _branch_as_chain(inp, j):
    """The same sequence cut to its prefix plus query j's branch, decoded as a
    single-query chain."""
    import types
    wl = inp.wl
    c, kr = inp.seq(0)
    L, Q = c.shape[0], wl.q_len
    rows = list(range(L - Q)) + [L - Q + i for i in _branch(inp.parents[0], j)]
    cw = wl.replace(q_len=1, seq_len=len(rows), tree=None)
    return types.SimpleNamespace(
        wl=cw, seq=lambda b: (c[rows], kr[rows]), parents=None, w_uk=inp.w_uk, w_uv=inp.w_uv,
        q_nope=inp.q_nope[:, j:j + 1], q_rope=inp.q_rope[:, j:j + 1])


def _q8_branches_ok(inp, tol=1e-12):
    ref = oracle.mla_decode_ref_q8(inp)
    ok = True
    for j in range(inp.wl.q_len):
        ch = oracle.mla_decode_ref_q8(_branch_as_chain(inp, j))
        for key in ("o", "o_lat"):
            a, b = ref[key][0, j], ch[key][0, 0]
            ok &= bool(np.max(np.abs(a - b)) <= tol * np.max(np.abs(b)))
        ok &= bool(abs(ref["lse"][0, j] - ch["lse"][0, 0]).max() <= tol * abs(ch["lse"]).max())
    return ok


@pytest.mark.parametrize("seed", range(4))
def test_q8_every_branch_equals_its_chain(seed):
    inp = _q8_tree_inputs(40 + seed)
    par = inp.parents[0]
    # the random tree must hold a token positioned before its slot, or the
    # pin would not tell slots from positions
    assert np.any(oracle.tree_depths(par) < np.arange(len(par)))
    assert _q8_branches_ok(inp)


def test_q8_tree_codes_keys_rotated_at_prefix_plus_depth():
    # the coded RoPE part of drafted token i is that of its raw key rotated at
    # L - Q + depth(i): equal to the chain-coded row of that position
    par = [-1, 0, 0, 1, -1, 4]
    inp = _q8_tree_inputs(5, parents=par)
    L, Q = 45, 6
    rows = oracle.mla_decode_ref_q8(inp)["rows"][0]
    c, kr = inp.seq(0)
    d = oracle.tree_depths(par)
    for i in range(Q):
        k = oracle.rotated_keys_f32(kr[L - Q + i:L - Q + i + 1], [L - Q + d[i]])
        r1, _, _ = oracle.quantize_cache_rows(c[L - Q + i:L - Q + i + 1], k)
        assert np.array_equal(rows["codes"][L - Q + i], r1["codes"][0])
        assert rows["rope_min"][L - Q + i] == r1["rope_min"][0]
        assert rows["rope_step"][L - Q + i] == r1["rope_step"][0]


def _q8_tree_battery():
    ok = True
    for seed in (60, 61):
        ok &= _q8_branches_ok(_q8_tree_inputs(seed))
    return bool(ok)


def _mut_keys_at_slots(seq_len, parents):
    # drafted keys rotated at their cache slot instead of prefix + depth
    _, qp = mla_ref._orig_positions(seq_len, parents)
    return np.arange(seq_len), qp


def _mut_queries_at_slots(seq_len, parents):
    kp, _ = mla_ref._orig_positions(seq_len, parents)
    return kp, seq_len - len(parents) + np.arange(len(parents))


def _mut_depth_plus_one(seq_len, parents):
    kp, qp = mla_ref._orig_positions(seq_len, parents)
    kp = kp.copy()
    kp[seq_len - len(parents):] += 1
    return kp, qp


@pytest.mark.parametrize("mutant", [_mut_keys_at_slots, _mut_queries_at_slots,
                                    _mut_depth_plus_one])
def test_planted_q8_tree_mistakes_are_caught(monkeypatch, mutant):
    assert _q8_tree_battery(), "clean oracle must pass the battery"
    monkeypatch.setattr(mla_ref, "_orig_positions", mla_ref.tree_positions, raising=False)
    monkeypatch.setattr(mla_ref, "tree_positions", mutant)
    assert not _q8_tree_battery(), "planted tree-position mistake went unnoticed"
