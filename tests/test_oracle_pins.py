"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: figures the
pages print (tests/golden/cache_accounting.txt), closed forms, identities that
must hold exactly (associativity, relative-position invariance, split + LSE
merge, verify == sequential decode), library routines (scipy's softmax and
logsumexp) and an independent pure-Python brute force on tiny inputs. The last
test plants plausible mistakes in the oracle and requires the battery to catch
every one of them.
"""
import math
import os

import numpy as np
import pytest
from scipy import special

import oracle
from oracle import brute, mla_ref
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_accounting.txt")
MiB, KiB, GiB = 2 ** 20, 2 ** 10, 2 ** 30


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, val, unit, src = [x.strip() for x in line.split("|")]
        assert src, name
        out[name] = int(val)
    return out


# ---------------------------------------------------------------- P1 accounting
def test_cache_accounting_matches_printed_figures():
    g = _golden()
    dc, dr = g["v2lite_kv_lora_rank"], g["v2lite_qk_rope_head_dim"]
    assert dc + dr == g["v2lite_latent_numbers_per_token_per_layer"]
    per_tok = oracle.latent_bytes_per_token(dc, dr, 2, g["v2lite_layers"])
    assert per_tok == g["v2lite_latent_bytes_per_token_all_layers"]
    assert per_tok * 32768 == g["v2lite_latent_mib_at_32768"] * MiB
    # the page puts vLLM's reservation within 0.01% of the calculation
    assert abs(per_tok - g["vllm_reserved_bytes_per_token"]) / per_tok < 1e-4
    plain = oracle.per_head_kv_bytes_per_token(g["v2lite_heads"], g["v2lite_key_width"],
                                               g["v2lite_value_width"], 2, g["v2lite_layers"])
    assert plain * 32768 == g["v2lite_plain_mib_at_32768"] * MiB
    assert round(plain / per_tok) == 9          # one ninth
    v3 = oracle.latent_bytes_per_token(512, 64, 2)
    assert v3 == g["v3_latent_bytes_per_token_per_layer"]
    v3_mha = oracle.per_head_kv_bytes_per_token(128, 128, 128, 2)
    assert v3_mha == g["v3_mha_equivalent_bytes_per_token_per_layer"]
    assert round(v3_mha / v3) == g["v3_compression_ratio_rounded"]
    kimi = oracle.latent_bytes_per_token(512, 64, 2, g["kimi_linear_mla_layers"]) * 32768
    assert kimi == g["kimi_linear_mla_mib_at_32768"] * MiB
    ll2 = oracle.per_head_kv_bytes_per_token(32, 128, 128, 2, 32)
    assert ll2 == g["llama2_7b_kib_per_token"] * KiB
    assert ll2 * 32768 == g["llama2_7b_gib_at_32768"] * GiB


# ---------------------------------------------------------------- P6 RoPE
def test_rope_closed_forms():
    base = 10000.0
    # d_r = 2: theta_0 = 1, so rotating (1, 0) by p gives (cos p, sin p)
    for p in [0, 1, 3, 1000, 1048575]:
        np.testing.assert_allclose(oracle.rope([1.0, 0.0], p, base), [math.cos(p), math.sin(p)],
                                   rtol=0, atol=1e-12)
    # d_r = 4: theta_1 = base^(-1/2) = 0.01, so the second pair turns by p/100
    out = oracle.rope([0.0, 0.0, 1.0, 0.0], 100, base)
    np.testing.assert_allclose(out, [0, 0, math.cos(1.0), math.sin(1.0)], atol=1e-14)
    # frequencies
    np.testing.assert_allclose(oracle.rope_freqs(8, base), [1, 0.1, 0.01, 0.001], rtol=1e-15)


def test_rope_rotation_properties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    pos = np.array([0, 7, 64, 32767, 1048575])
    y = oracle.rope(x, pos)
    # norm-preserving
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # composition R_a R_b = R_{a+b}, and R_{-p} R_p = I
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, 5), 11), oracle.rope(x, 16), atol=1e-12)
    np.testing.assert_allclose(oracle.rope(y, -pos), x, atol=1e-9)
    # each pair is a plane rotation: 2x2 matrix [[c, -s], [s, c]]
    th = oracle.rope_freqs(64)
    for i in [0, 5, 31]:
        a = 7 * th[i]
        rot = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
        np.testing.assert_allclose(oracle.rope(x[1], 7)[2 * i:2 * i + 2], rot @ x[1, 2 * i:2 * i + 2],
                                   atol=1e-13)


def test_rope_scores_depend_only_on_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    ref = oracle.rope(q, 900) @ oracle.rope(k, 500)
    for shift in [1, 1000, 500000]:
        np.testing.assert_allclose(oracle.rope(q, 900 + shift) @ oracle.rope(k, 500 + shift), ref,
                                   rtol=1e-10)


def test_rope_does_not_commute_with_a_projection():
    # R_pos(W^T a) != W^T R_pos(a): why the positional key is kept apart
    # ("The Architecture of Memory", "Decoupled Rotary Positional Encoding (RoPE)")
    rng = np.random.default_rng(3)
    W = rng.standard_normal((64, 64)) / 8
    a = rng.standard_normal(64)
    lhs = oracle.rope(W.T @ a, 37)
    rhs = W.T @ oracle.rope(a, 37)
    assert np.max(np.abs(lhs - rhs)) > 1e-3


# ---------------------------------------------------------------- P7 brute force
def _tiny_case(seed, B=2, H=2, dc=8, dr=4, dn=4, dv=4, Q=2, lens=(5, 6)):
    rng = np.random.default_rng(seed)
    w_uk = rng.standard_normal((H, dn, dc)) / math.sqrt(dc)
    w_uv = rng.standard_normal((H, dv, dc)) / math.sqrt(dc)
    seqs = []
    for b in range(B):
        L = lens[b]
        seqs.append(dict(c=rng.standard_normal((L, dc)), kr=rng.standard_normal((L, dr)),
                         qn=rng.standard_normal((Q, H, dn)), qr=rng.standard_normal((Q, H, dr))))
    return w_uk, w_uv, seqs, 1.0 / math.sqrt(dn + dr)


def _cmp_brute(w_uk, w_uv, s, scale, base=10000.0, tol=1e-12):
    o, ol, lse = oracle.attend_sequence(s["c"], s["kr"], s["qn"], s["qr"], w_uk, w_uv, scale, base, chunk=3)
    bo, bol, blse = brute.brute_sequence(s["c"].tolist(), s["kr"].tolist(), s["qn"].tolist(),
                                         s["qr"].tolist(), w_uk.tolist(), w_uv.tolist(), scale, base)
    ok = (np.allclose(o, bo, rtol=0, atol=tol * max(1.0, np.abs(bo).max()))
          and np.allclose(ol, bol, rtol=0, atol=tol * max(1.0, np.abs(bol).max()))
          and np.allclose(lse, blse, rtol=0, atol=tol * max(1.0, np.abs(blse).max())))
    return ok


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_brute_force_agrees(seed):
    w_uk, w_uv, seqs, scale = _tiny_case(seed)
    for s in seqs:
        assert _cmp_brute(w_uk, w_uv, s, scale)


def test_brute_force_agrees_single_query_long_positions():
    # positions far from zero exercise the RoPE angles
    w_uk, w_uv, seqs, scale = _tiny_case(9, B=1, Q=1, lens=(6,))
    s = seqs[0]
    assert _cmp_brute(w_uk, w_uv, s, scale, base=10000.0)
    assert _cmp_brute(w_uk, w_uv, s, scale, base=50.0)


# ---------------------------------------------------------------- P2 absorption
def test_absorbed_equals_unabsorbed():
    wl = workload.WORKLOADS["tiny_f32"]
    inp = workload.make(wl, 0)
    c, kr = inp.seq(0)
    o, ol, lse = oracle.attend_sequence(c, kr, inp.q_nope[0], inp.q_rope[0], inp.w_uk, inp.w_uv,
                                        wl.softmax_scale, wl.rope_base)
    ao, aol, alse = oracle.absorbed_attend_sequence(c, kr, inp.q_nope[0], inp.q_rope[0], inp.w_uk,
                                                    inp.w_uv, wl.softmax_scale, wl.rope_base)
    np.testing.assert_allclose(o, ao, rtol=1e-12, atol=1e-12 * np.abs(o).max())
    np.testing.assert_allclose(ol, aol, rtol=1e-12, atol=1e-12 * np.abs(ol).max())
    np.testing.assert_allclose(lse, alse, rtol=1e-12)


def test_absorbed_equals_unabsorbed_v2lite_shape_q4():
    wl = workload.WORKLOADS["v2lite_32k"].replace(batch=1, q_len=4, seq_len=200)
    inp = workload.make(wl, 5)
    c, kr = inp.seq(0)
    o, ol, lse = oracle.attend_sequence(c, kr, inp.q_nope[0], inp.q_rope[0], inp.w_uk, inp.w_uv,
                                        wl.softmax_scale, wl.rope_base, chunk=64)
    ao, aol, alse = oracle.absorbed_attend_sequence(c, kr, inp.q_nope[0], inp.q_rope[0], inp.w_uk,
                                                    inp.w_uv, wl.softmax_scale, wl.rope_base)
    np.testing.assert_allclose(o, ao, rtol=0, atol=1e-12 * np.abs(o).max())
    np.testing.assert_allclose(lse, alse, rtol=1e-12)


# ---------------------------------------------------------------- P3, P4 special cases
def test_single_cached_token_returns_v0():
    rng = np.random.default_rng(4)
    H, dn, dv, dc, dr = 3, 8, 8, 16, 8
    w_uk = rng.standard_normal((H, dn, dc))
    w_uv = rng.standard_normal((H, dv, dc))
    c, kr = rng.standard_normal((1, dc)), rng.standard_normal((1, dr))
    qn, qr = rng.standard_normal((1, H, dn)), rng.standard_normal((1, H, dr))
    o, ol, lse = oracle.attend_sequence(c, kr, qn, qr, w_uk, w_uv, 0.25)
    for h in range(H):
        np.testing.assert_allclose(o[0, h], w_uv[h] @ c[0], rtol=1e-15, atol=1e-14)
        np.testing.assert_allclose(ol[0, h], c[0], rtol=0, atol=0)
        # lse = the one score; position 0 means no rotation at all
        np.testing.assert_allclose(lse[0, h], 0.25 * (qn[0, h] @ (w_uk[h] @ c[0]) + qr[0, h] @ kr[0]),
                                   rtol=1e-13)


def test_zero_query_gives_mean_value():
    rng = np.random.default_rng(5)
    H, dn, dv, dc, dr, L = 2, 8, 6, 16, 8, 37
    w_uk = rng.standard_normal((H, dn, dc))
    w_uv = rng.standard_normal((H, dv, dc))
    c, kr = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    o, ol, lse = oracle.attend_sequence(c, kr, np.zeros((1, H, dn)), np.zeros((1, H, dr)),
                                        w_uk, w_uv, 0.3, chunk=8)
    for h in range(H):
        np.testing.assert_allclose(o[0, h], w_uv[h] @ c.mean(0), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(ol[0, h], c.mean(0), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(L), rtol=1e-14)


# ---------------------------------------------------------------- P5 scores / softmax
def test_score_is_content_plus_position_and_softmax_matches_scipy():
    rng = np.random.default_rng(6)
    H, dn, dv, dc, dr, L, Q = 2, 8, 8, 16, 8, 29, 3
    w_uk = rng.standard_normal((H, dn, dc)) / 4
    w_uv = rng.standard_normal((H, dv, dc)) / 4
    c, kr = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    qn, qr = rng.standard_normal((Q, H, dn)), rng.standard_normal((Q, H, dr))
    s = oracle.attend_scores(c, kr, qn, qr, w_uk, 0.2, chunk=5)
    o, ol, lse = oracle.attend_sequence(c, kr, qn, qr, w_uk, w_uv, 0.2, chunk=5)
    for j in range(Q):
        p = L - Q + j
        for h in range(H):
            content = np.array([qn[j, h] @ (w_uk[h] @ c[t]) for t in range(p + 1)])
            position = np.array([oracle.rope(qr[j, h], p) @ oracle.rope(kr[t], t) for t in range(p + 1)])
            np.testing.assert_allclose(s[j, h, :p + 1], 0.2 * (content + position), rtol=1e-13, atol=1e-13)
            assert np.all(np.isneginf(s[j, h, p + 1:]))
            w = special.softmax(s[j, h, :p + 1])
            np.testing.assert_allclose(ol[j, h], w @ c[:p + 1], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[j, h], special.logsumexp(s[j, h, :p + 1]), rtol=1e-13)


# ---------------------------------------------------------------- P8 split + LSE
def test_split_bounds_invariants():
    for L in [1, 63, 64, 65, 256, 1000, 32768, 1048576]:
        for S in [1, 2, 3, 7, 32, 64, 256]:
            b = oracle.split_bounds(L, S, 64)
            assert len(b) == S
            cov = [t for (a, e) in b for t in range(a, e)] if L <= 4096 else None
            if cov is not None:
                assert cov == list(range(L))
            assert b[0][0] == 0 and max(e for _, e in b) == L
            for (a, e), (a2, _) in zip(b, b[1:]):
                assert e == a2 or a2 == L
                assert a % 64 == 0 or a == L


def test_split_bounds_fixed_chunk():
    # every sequence is cut at multiples of the same chunk; units past its end are empty
    for L in [1, 63, 64, 65, 383, 384, 385, 1000, 32768]:
        for chunk in [64, 128, 384]:
            S = -(-32768 // chunk)
            b = oracle.split_bounds(L, S, 64, chunk)
            assert len(b) == S
            assert [(a, e) for a, e in b if e > a] == [(a, min(L, a + chunk))
                                                       for a in range(0, L, chunk)]
            assert all(e - a <= chunk for a, e in b)
            assert all(a == e == L for a, e in b[-(-L // chunk):])


@pytest.mark.parametrize("L,S,chunk", [(256, 1, 0), (256, 4, 0), (200, 7, 0), (65, 3, 0),
                                       (64, 64, 0), (300, 2, 0), (300, 8, 64), (130, 5, 64)])
def test_split_merge_equals_unsplit(L, S, chunk):
    rng = np.random.default_rng(L * 31 + S)
    H, dn, dc, dr, Q = 3, 8, 16, 8, 2
    w_uk = rng.standard_normal((H, dn, dc)) / 4
    w_uv = rng.standard_normal((H, 8, dc)) / 4
    c, kr = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    qn, qr = rng.standard_normal((Q, H, dn)), rng.standard_normal((Q, H, dr))
    o, ol, lse = oracle.attend_sequence(c, kr, qn, qr, w_uk, w_uv, 0.3)
    op, lp = oracle.attend_partials(c, kr, qn, qr, w_uk, 0.3, S, chunk_tokens=chunk)
    mo, ml = oracle.lse_combine(op, lp)
    np.testing.assert_allclose(mo, ol, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml, lse, rtol=1e-13)
    if S == 1:
        np.testing.assert_allclose(op[:, :, 0], ol, rtol=1e-13, atol=1e-14)


def test_lse_combine_algebra():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((4, 16))
    l = rng.standard_normal(4)
    # a -inf split contributes nothing
    o2 = np.concatenate([o, rng.standard_normal((1, 16))])
    l2 = np.concatenate([l, [-np.inf]])
    a, la = oracle.lse_combine(o, l)
    b, lb = oracle.lse_combine(o2, l2)
    np.testing.assert_allclose(a, b, rtol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-15)
    # two identical halves: same output, lse + ln 2
    c, lc = oracle.lse_combine(np.stack([o[0], o[0]]), np.array([l[0], l[0]]))
    np.testing.assert_allclose(c, o[0], rtol=1e-15)
    np.testing.assert_allclose(lc, l[0] + math.log(2), rtol=1e-15)
    # matches scipy's logsumexp
    np.testing.assert_allclose(la, special.logsumexp(l), rtol=1e-15)


# ---------------------------------------------------------------- P9 verify
def test_verify_equals_sequential_decode():
    rng = np.random.default_rng(8)
    H, dn, dv, dc, dr, L, Q = 2, 8, 8, 16, 8, 41, 4
    w_uk = rng.standard_normal((H, dn, dc)) / 4
    w_uv = rng.standard_normal((H, dv, dc)) / 4
    c, kr = rng.standard_normal((L, dc)), rng.standard_normal((L, dr))
    qn, qr = rng.standard_normal((Q, H, dn)), rng.standard_normal((Q, H, dr))
    o, ol, lse = oracle.attend_sequence(c, kr, qn, qr, w_uk, w_uv, 0.3, chunk=16)
    for j in range(Q):
        Lj = L - Q + j + 1
        oj, olj, lj = oracle.attend_sequence(c[:Lj], kr[:Lj], qn[j:j + 1], qr[j:j + 1], w_uk, w_uv, 0.3)
        np.testing.assert_allclose(o[j], oj[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[j], lj[0], rtol=1e-14)


# ---------------------------------------------------------------- append image
def test_cache_append_round_trip_through_page_table():
    wl = workload.WORKLOADS["v2lite_paged_varlen"].replace(batch=3, len_range=(1, 200))
    inp = workload.make(wl, 11)
    D = wl.dim
    poison = np.uint16(0x7FC1)
    pool = np.full((inp.num_pages, 64, D), poison, dtype=np.uint16)
    bits_c = workload.bf16_bits(inp.c)
    bits_k = workload.bf16_bits(inp.k_rope)
    seq_idx = np.concatenate([np.full(L, b) for b, L in enumerate(inp.seq_lens)])
    pos = np.concatenate([np.arange(L) for L in inp.seq_lens])
    img = oracle.cache_append_image(pool, bits_c, bits_k, seq_idx, pos, inp.page_table, wl.kv_rank)
    flat = img.reshape(-1, D)
    written = np.zeros(flat.shape[0], bool)
    for b, L in enumerate(inp.seq_lens):
        for t in range(L):
            slot = inp.page_table[b][t // 64] * 64 + t % 64
            row = flat[slot]
            n = inp.offsets[b] + t
            assert np.array_equal(row[:wl.kv_rank], bits_c[n]) and np.array_equal(row[wl.kv_rank:], bits_k[n])
            written[slot] = True
    assert written.sum() == int(inp.seq_lens.sum())
    assert np.all(flat[~written] == poison)
    assert np.array_equal(pool, np.full_like(pool, poison))   # input untouched


def test_cache_append_rotate_mode_stores_rotated_key():
    pt = np.array([[1, 0]], dtype=np.int32)
    pool = np.zeros((2, 64, 6))
    c = np.array([[1.0, 2.0]])
    kr = np.array([[1.0, 0.0, 0.0, 1.0]])
    img = oracle.cache_append_image(pool, c, kr, [0], [70], pt, 2, rotate=True)
    row = img[0, 6]                                  # page_table[0][1] = 0, slot 70 % 64
    np.testing.assert_allclose(row[:2], [1, 2])
    np.testing.assert_allclose(row[2:], [math.cos(70), math.sin(70), -math.sin(0.7), math.cos(0.7)],
                               atol=1e-14)


# ---------------------------------------------------------------- planted mistakes
def _battery():
    """The pins above, compressed: True when the oracle passes all of them."""
    ok = True
    for seed in [0, 1]:
        w_uk, w_uv, seqs, scale = _tiny_case(seed)
        for s in seqs:
            ok &= _cmp_brute(w_uk, w_uv, s, scale)
    rng = np.random.default_rng(4)
    H, dn, dv, dc, dr = 2, 4, 4, 8, 4
    w_uk = rng.standard_normal((H, dn, dc))
    w_uv = rng.standard_normal((H, dv, dc))
    c, kr = rng.standard_normal((1, dc)), rng.standard_normal((1, dr))
    o, _, _ = oracle.attend_sequence(c, kr, rng.standard_normal((1, H, dn)),
                                     rng.standard_normal((1, H, dr)), w_uk, w_uv, 0.25)
    ok &= all(np.allclose(o[0, h], w_uv[h] @ c[0]) for h in range(H))
    return bool(ok)


def _mut_rope_sign(x, pos, base=10000.0):
    return mla_ref._orig_rope(x, -np.asarray(pos, float), base)


def _mut_rope_halves(x, pos, base=10000.0):
    x = np.asarray(x, float)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    y = mla_ref._orig_rope(x[..., inv], pos, base)
    return y[..., perm]


def _mut_positions(L, Q):
    return np.full(Q, L - 1)


def _mut_positions_off(L, Q):
    return L - Q + np.arange(Q) - 1


def _mut_expand_swap(c, kr, positions, w_uk, w_uv=None, base=10000.0):
    # value weights of the wrong head
    wv = None if w_uv is None else np.asarray(w_uv)[::-1]
    return mla_ref._orig_expand(c, kr, positions, w_uk, wv, base)


def _mut_expand_norope(c, kr, positions, w_uk, w_uv=None, base=10000.0):
    return mla_ref._orig_expand(c, kr, None if positions is None else np.zeros_like(positions),
                                w_uk, w_uv, base)


def _mut_expand_transpose(c, kr, positions, w_uk, w_uv=None, base=10000.0):
    # uses the wrong slice orientation of a square per-head block
    wk = None if w_uk is None else np.asarray(w_uk)[:, :, ::-1]
    return mla_ref._orig_expand(c, kr, positions, wk, w_uv, base)


@pytest.mark.parametrize("target,mutant", [
    ("rope", _mut_rope_sign),
    ("rope", _mut_rope_halves),
    ("query_positions", _mut_positions),
    ("query_positions", _mut_positions_off),
    ("expand_kv", _mut_expand_swap),
    ("expand_kv", _mut_expand_norope),
    ("expand_kv", _mut_expand_transpose),
])
def test_planted_mistakes_are_caught(monkeypatch, target, mutant):
    assert _battery(), "clean oracle must pass the battery"
    monkeypatch.setattr(mla_ref, "_orig_rope", mla_ref.rope, raising=False)
    monkeypatch.setattr(mla_ref, "_orig_expand", mla_ref.expand_kv, raising=False)
    monkeypatch.setattr(mla_ref, target, mutant)
    assert not _battery(), f"planted mistake in {target} went unnoticed"


def test_planted_scale_and_mask_mistakes_are_caught(monkeypatch):
    orig = mla_ref.attend_scores

    def no_scale(c, kr, qn, qr, w_uk, scale, base=10000.0, chunk=1024, parents=None):
        return orig(c, kr, qn, qr, w_uk, 1.0, base, chunk, parents=parents)

    monkeypatch.setattr(mla_ref, "attend_scores", no_scale)
    assert not _battery()
    monkeypatch.setattr(mla_ref, "attend_scores", orig)
    monkeypatch.setattr(mla_ref, "causal_mask", lambda L, pq: np.zeros((len(pq), L), bool))
    assert not _battery()
    monkeypatch.setattr(mla_ref, "causal_mask",
                        lambda L, pq: np.arange(L)[None, :] >= np.asarray(pq)[:, None])
    assert not _battery()
