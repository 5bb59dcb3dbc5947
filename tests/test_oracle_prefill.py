"""Pins of the oracle's chunked prefill against what fixes it independently.

Chunked prefill ("Beyond the Attention Bottleneck", "Chunked Prefilling"): a
long prompt is split into chunks processed one after another, each chunk's
tokens joining the cache before its queries attend to it. The split bounds
the memory of a prefill step; it must not change what attention computes,
so the pins are: any chunk size gives one-shot causal attention over the
whole prompt, chunk 1 is token-by-token decode, a scalar-loop brute force on
tiny prompts, a prefill that starts after an already cached prefix, and
planted mistakes (a chunk that does not see itself, a chunk that sees the
whole prompt, queries positioned from the chunk start) that the battery
must catch.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import brute, mla_ref


def _prompt(seed, N=23, H=2, dn=4, dv=4, dc=8, dr=4):
    rng = np.random.default_rng(seed)
    return dict(c=rng.standard_normal((N, dc)), kr=rng.standard_normal((N, dr)),
                qn=rng.standard_normal((N, H, dn)), qr=rng.standard_normal((N, H, dr)),
                w_uk=rng.standard_normal((H, dn, dc)) / math.sqrt(dc),
                w_uv=rng.standard_normal((H, dv, dc)) / math.sqrt(dc),
                scale=1.0 / math.sqrt(dn + dr))


def _chunked(k, chunk, cached=0):
    return oracle.prefill_in_chunks(k["c"], k["kr"], k["qn"][cached:], k["qr"][cached:],
                                    k["w_uk"], k["w_uv"], k["scale"], chunk, cached=cached)


def _one_shot(k, cached=0):
    # the whole prompt as one Q = N - cached chain over the full cache
    return oracle.attend_sequence(k["c"], k["kr"], k["qn"][cached:], k["qr"][cached:], k["w_uk"],
                                  k["w_uv"], k["scale"])


def _close(a, b, tol=1e-12):
    return all(np.allclose(x, y, rtol=0, atol=tol * max(1.0, np.abs(y).max()))
               for x, y in zip(a, b))


def _brute_ok(seed, chunk, cached=0):
    k = _prompt(seed, N=9)
    got = _chunked(k, chunk, cached)
    ref = brute.brute_sequence(k["c"].tolist(), k["kr"].tolist(), k["qn"][cached:].tolist(),
                               k["qr"][cached:].tolist(), k["w_uk"].tolist(),
                               k["w_uv"].tolist(), k["scale"])
    return _close(got, [np.asarray(r) for r in ref])


@pytest.mark.parametrize("chunk", [1, 2, 5, 8, 23, 64])
def test_any_chunk_size_is_one_shot_causal_attention(chunk):
    for seed in range(3):
        k = _prompt(seed)
        assert _close(_chunked(k, chunk), _one_shot(k))


def test_chunk_one_is_token_by_token_decode():
    k = _prompt(4, N=12)
    o, ol, lse = _chunked(k, 1)
    for i in range(12):   # query i decodes over tokens 0..i with Q = 1
        oi, oli, li = oracle.attend_sequence(k["c"][:i + 1], k["kr"][:i + 1], k["qn"][i:i + 1],
                                             k["qr"][i:i + 1], k["w_uk"], k["w_uv"], k["scale"])
        assert np.allclose(o[i], oi[0], rtol=0, atol=1e-13) and np.allclose(lse[i], li[0])


@pytest.mark.parametrize("chunk,cached", [(1, 0), (3, 0), (4, 2), (9, 5)])
def test_brute_force_with_and_without_a_cached_prefix(chunk, cached):
    for seed in range(2):
        assert _brute_ok(100 + seed, chunk, cached)


def test_prefill_after_a_cached_prefix_equals_the_tail_of_one_shot():
    k = _prompt(7, N=30)
    full = _one_shot(k)
    tail = _chunked(k, 6, cached=11)
    assert _close(tail, tuple(x[11:] for x in full))


# ---------------------------------------------------------------- planted mistakes
def _battery():
    ok = True
    for seed in (200, 201):
        k = _prompt(seed)
        ok &= _close(_chunked(k, 5), _one_shot(k))
        ok &= _brute_ok(seed, 4) and _brute_ok(seed, 3, cached=2)
    return bool(ok)


def _mut_chunk_blind_to_itself(c, kr, qn, qr, w_uk, w_uv, scale, chunk, base=10000.0, cached=0):
    # each chunk attends only to the cache before it (plus its first token)
    N = len(c)
    outs = []
    for s in range(cached, N, chunk):
        e = min(N, s + chunk)
        rows = [mla_ref.attend_sequence(c[:s + 1], kr[:s + 1], qn[i - cached:i - cached + 1],
                                        qr[i - cached:i - cached + 1], w_uk, w_uv, scale, base)
                for i in range(s, e)]
        outs.extend(rows)
    return tuple(np.concatenate([o[i] for o in outs]) for i in range(3))


def _mut_sees_whole_prompt(c, kr, qn, qr, w_uk, w_uv, scale, chunk, base=10000.0, cached=0):
    N = len(c)
    outs = []
    for s in range(cached, N, chunk):
        e = min(N, s + chunk)
        # queries of the chunk placed at the end of the prompt: they see it all
        o = mla_ref.attend_sequence(c, kr, qn[s - cached:e - cached], qr[s - cached:e - cached],
                                    w_uk, w_uv, scale, base)
        outs.append(o)
    return tuple(np.concatenate([o[i] for o in outs]) for i in range(3))


def _mut_positions_from_chunk_start(c, kr, qn, qr, w_uk, w_uv, scale, chunk, base=10000.0,
                                    cached=0):
    N = len(c)
    outs = []
    for s in range(cached, N, chunk):
        e = min(N, s + chunk)
        # the chunk's tokens re-numbered from 0 (keys and queries), prefix dropped
        outs.append(mla_ref.attend_sequence(c[s:e], kr[s:e], qn[s - cached:e - cached],
                                            qr[s - cached:e - cached], w_uk, w_uv, scale, base))
    return tuple(np.concatenate([o[i] for o in outs]) for i in range(3))


@pytest.mark.parametrize("mutant", [_mut_chunk_blind_to_itself, _mut_sees_whole_prompt,
                                    _mut_positions_from_chunk_start])
def test_planted_prefill_mistakes_are_caught(monkeypatch, mutant):
    assert _battery(), "clean oracle must pass the battery"
    monkeypatch.setattr(mla_ref, "prefill_in_chunks", mutant)
    monkeypatch.setattr(oracle, "prefill_in_chunks", mutant)
    assert not _battery(), "planted mistake in prefill_in_chunks went unnoticed"
