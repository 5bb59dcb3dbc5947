"""Pins of the oracle's 4-bit latent cache against what fixes it independently.

The listing of "KV Cache Optimization: Scaling to Million-Token Contexts"
(technique 3) codes each cached row between its own minimum and maximum and
defaults to 4 bits; the comparison table puts INT4 at 4x less memory. The
4-bit cache keeps the 8-bit cache's per-row coding with 16 levels and packs
two codes per byte. Pins: the quantizer's properties and closed forms at 16
levels, the nibble packing (closed form, round trip), lossless rows giving
exactly the unquantized attention, the coding error bracketed between the
8-bit one and a few percent, drafted trees (every branch equals its chain),
and planted mistakes the battery must catch.
"""
import math
import types

import numpy as np
import pytest

import oracle
from oracle import mla_ref
import workload


def _rows(seed, n=12, d=512):
    rng = np.random.default_rng(seed)
    out = [rng.standard_normal(d).astype(np.float32),
           (rng.standard_normal(d) * 40 + 7).astype(np.float32),
           rng.uniform(-1e-3, 1e-3, d).astype(np.float32),
           np.where(rng.random(d) < 0.02, 30.0, rng.standard_normal(d)).astype(np.float32)]
    out.extend((rng.standard_normal((n, d)) * rng.uniform(0.1, 5, (n, 1))).astype(np.float32))
    return out


def _quantizer_ok(x):
    q, mn, step = oracle.quantize_q4(x)
    x = np.asarray(x, np.float64)
    if step == 0:
        return bool(np.all(q == 0))
    deq = oracle.dequantize_q8(q, mn, step)
    ok = np.max(np.abs(deq - x)) <= step * (0.5 + 1e-4)            # within half a step
    ok &= q[np.argmin(x)] == 0 and q[np.argmax(x)] == oracle.Q4_LEVELS  # extremes
    ok &= int(q.max()) <= 15
    order = np.argsort(x, kind="stable")
    ok &= bool(np.all(np.diff(q[order].astype(int)) >= 0))        # monotone
    ok &= float(mn) == x.min()                                      # the range starts at the min
    ok &= abs(float(mn) + 15 * float(step) - x.max()) <= 1e-5 * max(1.0, abs(x.max()))
    return bool(ok)


@pytest.mark.parametrize("seed", range(3))
def test_quantizer_properties(seed):
    for x in _rows(seed):
        assert _quantizer_ok(x)


def test_quantizer_and_packing_closed_forms():
    q, mn, step = oracle.quantize_q4(np.arange(16, dtype=np.float32))   # step exactly 1
    assert mn == 0 and step == 1 and np.array_equal(q, np.arange(16))
    q, mn, step = oracle.quantize_q4(np.array([-1.0, 1.0, 0.0], np.float32))
    assert q[0] == 0 and q[1] == 15 and step == np.float32(2 / 15) and q[2] in (7, 8)
    q, mn, step = oracle.quantize_q4(np.full(5, -3.5, np.float32))
    assert step == 0 and np.all(q == 0) and mn == -3.5
    # column 2i in the low nibble of byte i, 2i + 1 in the high nibble
    packed = oracle.pack_q4(np.arange(16, dtype=np.uint8))
    assert packed.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (7, 576)).astype(np.uint8)
    assert oracle.pack_q4(codes).shape == (7, 288)
    assert np.array_equal(oracle.unpack_q4(oracle.pack_q4(codes)), codes)


def _lossless_case(seed, L=40, Q=3, H=2, dn=8, dv=8, dc=32, dr=8):
    """Rows whose parts are exactly mn + code * step with codes 0 and 15
    present and power-of-two steps: 4-bit coding loses nothing on them."""
    rng = np.random.default_rng(seed)

    def exact_part(n):
        codes = rng.integers(0, 16, n)
        codes[0] = 0
        codes[-1] = 15
        rng.shuffle(codes)
        step = 2.0 ** -int(rng.integers(2, 7))
        mn = step * int(rng.integers(-40, 40))
        return (mn + codes * step).astype(np.float32)

    c = np.stack([exact_part(dc) for _ in range(L)])
    kr = np.stack([exact_part(dr) for _ in range(L)])
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    qn, qr = rng.standard_normal((Q, H, dn)), rng.standard_normal((Q, H, dr))
    return c, kr, qn, qr, w_uk, w_uv, 1.0 / math.sqrt(dn + dr)


def test_lossless_rows_give_the_unquantized_attention():
    for seed in range(3):
        c, kr, qn, qr, w_uk, w_uv, sc = _lossless_case(seed)
        rows, c_hat, k_hat = oracle.quantize_cache_rows(c, kr, bits=4)
        assert np.array_equal(c_hat, c.astype(np.float64))
        assert np.array_equal(k_hat, kr.astype(np.float64))
        assert rows["codes"].max() == 15
        o, ol, lse = oracle.attend_sequence_rotated(c_hat, k_hat, qn, qr, w_uk, w_uv, sc)
        o2, ol2, lse2 = oracle.attend_sequence_rotated(c, kr, qn, qr, w_uk, w_uv, sc)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_q4_error_between_q8_and_a_bound():
    # 16 levels per row part: coarser than 8 bits, yet near the exact attention
    wl = workload.WORKLOADS["v2lite_32k"].replace(batch=2, seq_len=300)
    inp = workload.make(wl, 1)
    ref = oracle.mla_decode_ref(inp)
    q8 = oracle.mla_decode_ref_q8(inp)
    q4 = oracle.mla_decode_ref_q4(inp)
    for key in ("o", "o_lat"):
        scale = np.abs(ref[key]).max()
        e8 = np.abs(q8[key] - ref[key]).max() / scale
        e4 = np.abs(q4[key] - ref[key]).max() / scale
        assert e8 < e4 < 0.25, (key, e8, e4)
    assert np.abs(q4["lse"] - ref["lse"]).max() < 0.25


# ---------------------------------------------------------------- drafted trees
def _tree_inputs(seed, L=45, Q=6):
    wl = workload.WORKLOADS["tiny_f32"].replace(q_len=Q, seq_len=L, tree="random", cache="q4")
    return workload.make(wl, seed)


def _branch(parents, j):
    path = []
    while j != -1:
        path.append(j)
        j = int(parents[j])
    return path[::-1]


def _branches_ok(inp, tol=1e-12):
    ref = oracle.mla_decode_ref_q4(inp)
    c, kr = inp.seq(0)
    L, Q = c.shape[0], inp.wl.q_len
    ok = True
    for j in range(Q):
        rows = list(range(L - Q)) + [L - Q + i for i in _branch(inp.parents[0], j)]
        ch_in = types.SimpleNamespace(
            wl=inp.wl.replace(q_len=1, seq_len=len(rows), tree=None),
            seq=lambda b, rows=rows: (c[rows], kr[rows]), parents=None, w_uk=inp.w_uk,
            w_uv=inp.w_uv, q_nope=inp.q_nope[:, j:j + 1], q_rope=inp.q_rope[:, j:j + 1])
        ch = oracle.mla_decode_ref_q4(ch_in)
        for key in ("o", "o_lat"):
            ok &= bool(np.max(np.abs(ref[key][0, j] - ch[key][0, 0]))
                       <= tol * np.max(np.abs(ch[key])))
        ok &= bool(np.abs(ref["lse"][0, j] - ch["lse"][0, 0]).max() <= tol * np.abs(ch["lse"]).max())
    return ok


@pytest.mark.parametrize("seed", range(3))
def test_q4_every_branch_equals_its_chain(seed):
    inp = _tree_inputs(70 + seed)
    assert np.any(oracle.tree_depths(inp.parents[0]) < np.arange(inp.wl.q_len))
    assert _branches_ok(inp)


# ---------------------------------------------------------------- planted mistakes
def _battery():
    ok = all(_quantizer_ok(x) for x in _rows(7, n=4))
    for seed in range(2):
        c, kr, qn, qr, w_uk, w_uv, sc = _lossless_case(seed)
        _, c_hat, k_hat = oracle.quantize_cache_rows(c, kr, bits=4)
        ok &= np.array_equal(c_hat, c.astype(np.float64)) and np.array_equal(k_hat, kr)
    packed = oracle.pack_q4(np.arange(16, dtype=np.uint8))
    ok &= packed.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    ok &= _branches_ok(_tree_inputs(80))
    return bool(ok)


def _q_floor(x):
    x = np.asarray(x, np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(15))
    if step == 0:
        return np.zeros(x.shape, np.uint8), mn, step
    return np.clip(np.floor((x - mn) / step), 0, 15).astype(np.uint8), mn, step


def _q_16(x):
    x = np.asarray(x, np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(16))
    if step == 0:
        return np.zeros(x.shape, np.uint8), mn, step
    return np.clip(np.rint((x - mn) / step), 0, 15).astype(np.uint8), mn, step


def _q_from_max(x):
    x = np.asarray(x, np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(15))
    if step == 0:
        return np.zeros(x.shape, np.uint8), mn, step
    return np.clip(np.rint((mx - x) / step), 0, 15).astype(np.uint8), mn, step


def _pack_swapped(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 1::2] | (codes[..., 0::2] << 4)).astype(np.uint8)


def _keys_at_slots(seq_len, parents):
    _, qp = mla_ref._orig_positions(seq_len, parents)
    return np.arange(seq_len), qp


@pytest.mark.parametrize("target,mutant", [
    ("quantize_q4", _q_floor),
    ("quantize_q4", _q_16),
    ("quantize_q4", _q_from_max),
    ("pack_q4", _pack_swapped),
    ("tree_positions", _keys_at_slots),
])
def test_planted_q4_mistakes_are_caught(monkeypatch, target, mutant):
    assert _battery(), "clean oracle must pass the battery"
    monkeypatch.setattr(mla_ref, "_orig_positions", mla_ref.tree_positions, raising=False)
    monkeypatch.setattr(mla_ref, target, mutant)
    monkeypatch.setattr(oracle, target, mutant)
    assert not _battery(), f"planted mistake in {target} went unnoticed"
