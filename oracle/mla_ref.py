"""fp64 CPU oracle for MLA decode over a latent KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its binding) never imports, links or calls it, and this
module imports nothing from the product path.

What it computes, and where the pages define it:

* Latent cache entry of one token and layer: a d_c-wide latent c_t plus a
  d_r-wide decoupled RoPE key, 576 numbers for the DeepSeek MLA shapes
  ("DeepSeek's Config Says 16 KV Heads, Its Cache Holds a Ninth of That",
  section 5 "Multi-head latent attention (MLA)"; "The Architecture of Memory",
  "Decoupled Rotary Positional Encoding (RoPE)").
* Up-projection K_t = W_UK c_t, V_t = W_UV c_t ("Beyond the Attention
  Bottleneck", "Down-Projection and Up-Projection Mechanics"), taken per head.
* The score of a query against a key is the sum of a content part (against
  the expanded key) and a positional part (against the RoPE key, shared by all
  heads) ("Beyond the Attention Bottleneck", "The RoPE Compatibility Problem";
  "The Architecture of Memory", "Decoupled Rotary Positional Encoding (RoPE)").
* Decode: the new token is appended, then its query attends over the whole
  cache ("The Architecture of Memory", "The Decode Phase: The Memory Bandwidth
  Wall"); several drafted tokens are verified in one pass and must agree with
  token-by-token decoding ("The Architecture of Memory", "Speculative
  Decoding: Amortizing the Memory Fetch").
* Tree verification: the drafted tokens form a tree whose branches must not
  see each other; the query of a drafted token attends to the whole prefix
  with no mask and to the drafted tokens on its own branch under a causal
  tree mask ("The Architecture of Memory", "Tree Attention Verification").
  Reading: a drafted token attached to the prefix sits at position
  L - Q, a child one position after its parent (position = L - Q + depth),
  for its query and its cached RoPE key alike, so that every branch is scored
  exactly as the chain of its tokens decoded one by one would be.
* A low-precision latent cache: rows quantized to 8 bits between their own
  minimum and maximum ("KV Cache Optimization: Scaling to Million-Token
  Contexts", technique 3 "KV Cache Quantization", and its comparison table:
  an INT8 cache halves the bytes). Reading: per cached token, separately for
  the latent part and the (rotated) RoPE part, in float32.
* Chunked prefill: the prompt enters the cache in chunks, each chunk's
  queries attending causally to everything cached so far ("Beyond the
  Attention Bottleneck", "Chunked Prefilling"); in the absorbed form a chunk
  of C tokens is the Q = C chain of the decode above.
* A sparse read: a small scorer rates every cached token and attention reads
  only the top-scored ones ("DeepSeek's Config Says 16 KV Heads, Its Cache
  Holds a Ninth of That", section 6, "Sparse attention"). Reading: the score
  is a weighted sum over the scorer's heads of ReLU(q . k), ties in the top-k
  go to the smaller token index.
* Split-KV partials merged by a log-sum-exp reduction ("The Architecture of
  Memory", "Flash-Decoding and FlashInfer").
* Paged cache: fixed-size pages mapped logical -> physical through a page
  table ("The Architecture of Memory", "PagedAttention: Virtual Memory for
  LLMs"; "KV Cache Optimization: Scaling to Million-Token Contexts",
  technique 7 "Paged Attention (vLLM)").

This oracle NEVER absorbs weights in ``attend_sequence``: it rebuilds every
head's K_t and V_t from the latent and runs textbook softmax attention. The
absorbed form exists only in ``absorbed_query`` / ``absorbed_attend_sequence``,
which the tests use to pin the associativity identity and to check the
query-absorption kernel.

Readings taken where the pages are silent (each is listed in the design notes):
RoPE rotates interleaved pairs (x_2i, x_2i+1) by pos * base^(-2i/d_r); the
cached RoPE key is stored rotated; query j of Q sits at position L - Q + j and
sees keys t <= L - Q + j; the softmax scale is 1/sqrt(d_n + d_r); only the d_c
latent columns enter the value side; logs are natural.

Pins (tests/test_oracle_pins.py): brute force in pure Python on tiny inputs,
absorbed == unabsorbed, L = 1 gives V_0, a zero query gives the mean value,
RoPE closed forms and relative-position invariance, any split merged by LSE
equals the unsplit result, Q-token verify equals sequential decode, cache
accounting against the figures the pages print, append round-trip through the
page table. No function here is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


# --------------------------------------------------------------------------
# cache accounting
# --------------------------------------------------------------------------
def latent_bytes_per_token(kv_rank: int, rope_dim: int, elem_bytes: int,
                           layers: int = 1) -> int:
    """Bytes one token adds to an MLA cache: one (d_c + d_r) row per layer.

    "DeepSeek's Config Says 16 KV Heads", introduction and section 5: 576
    numbers x 2 bytes x 27 layers for V2-Lite.
    """
    return (kv_rank + rope_dim) * elem_bytes * layers


def per_head_kv_bytes_per_token(heads: int, key_dim: int, value_dim: int,
                                elem_bytes: int, layers: int = 1) -> int:
    """Bytes one token would add if every head kept its own key and value.

    "DeepSeek's Config Says 16 KV Heads", introduction ((192 + 128) x 16 heads x
    2 bytes x 27 layers for V2-Lite); "The Architecture of Memory", "DeepSeek's
    Multi-Head Latent Attention (MLA)" (MHA-equivalent footprint for V3).
    """
    return (key_dim + value_dim) * heads * elem_bytes * layers


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def rope_freqs(rope_dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base^(-2i/d_r), i = 0 .. d_r/2 - 1 (fp64)."""
    i = np.arange(rope_dim // 2, dtype=F64)
    return np.power(F64(base), -2.0 * i / rope_dim)


def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate interleaved pairs of the last axis of ``x`` by pos * theta_i.

    ``pos`` broadcasts against ``x.shape[:-1]``. Angles are formed in fp64.
    The rotation is the position-dependent one the pages require to be applied
    to the positional query/key parts only ("The Architecture of Memory",
    "Decoupled Rotary Positional Encoding (RoPE)").
    """
    x = np.asarray(x, dtype=F64)
    pos = np.asarray(pos, dtype=F64)
    ang = pos[..., None] * rope_freqs(x.shape[-1], base)
    cs, sn = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (x.shape[-1],)), F64)
    out[..., 0::2] = x0 * cs - x1 * sn
    out[..., 1::2] = x0 * sn + x1 * cs
    return out


# --------------------------------------------------------------------------
# unabsorbed attention (the oracle proper)
# --------------------------------------------------------------------------
def expand_kv(c, k_rope_raw, positions, w_uk, w_uv=None, base: float = 10000.0):
    """Per-head keys and values rebuilt from cached latents.

    K_t,h = [W_UK[h] c_t ; RoPE(k^R_t, t)] (the RoPE key shared by all heads),
    V_t,h = W_UV[h] c_t ("Beyond the Attention Bottleneck", "Down-Projection
    and Up-Projection Mechanics" and "The RoPE Compatibility Problem").
    Returns K [T][H][d_n + d_r] (None when ``w_uk`` is None) and V [T][H][d_v]
    (None when ``w_uv`` is None).
    """
    c = np.asarray(c, F64)
    T = c.shape[0]
    k = None
    if w_uk is not None:
        w_uk = np.asarray(w_uk, F64)
        H, dn, dc = w_uk.shape
        kc = (c @ w_uk.reshape(H * dn, dc).T).reshape(T, H, dn)
        kr = rope(k_rope_raw, positions, base)
        k = np.concatenate([kc, np.broadcast_to(kr[:, None, :], (T, H, kr.shape[-1]))], axis=-1)
    v = None
    if w_uv is not None:
        w_uv = np.asarray(w_uv, F64)
        Hv, dv, dcv = w_uv.shape
        v = (c @ w_uv.reshape(Hv * dv, dcv).T).reshape(T, Hv, dv)
    return k, v


def query_positions(seq_len: int, q_len: int) -> np.ndarray:
    """Drafted/current query j sits at L - Q + j (appended before attending)."""
    return seq_len - q_len + np.arange(q_len)


def tree_depths(parents) -> np.ndarray:
    """Depth of each drafted token: 0 when its parent is -1 (attached to the
    prefix), else one more than its parent's. Parents precede their children."""
    parents = [int(p) for p in parents]
    depth = np.zeros(len(parents), dtype=np.int64)
    for j, p in enumerate(parents):
        if not -1 <= p < j:
            raise ValueError(f"drafted token {j} has parent {p}: parents must precede children")
        depth[j] = 0 if p < 0 else depth[p] + 1
    return depth


def tree_ancestry(parents) -> np.ndarray:
    """[Q][Q] bool: entry (j, i) is True when drafted token i is j itself or one
    of its ancestors, i.e. when i lies on j's branch ("Tree Attention
    Verification": independent branches do not attend to one another)."""
    Q = len(parents)
    tree_depths(parents)  # validates the order
    anc = np.zeros((Q, Q), dtype=bool)
    for j in range(Q):
        i = j
        while i >= 0:
            anc[j, i] = True
            i = int(parents[i])
    return anc


def tree_positions(seq_len: int, parents):
    """(key positions [L], query positions [Q]) with a drafted tree: prefix
    token t keeps position t, drafted token i (cached at slot L - Q + i) and
    its query sit at L - Q + depth(i)."""
    Q = len(parents)
    pre = seq_len - Q
    d = tree_depths(parents)
    kp = np.arange(seq_len, dtype=np.int64)
    kp[pre:] = pre + d
    return kp, pre + d


def tree_excluded(seq_len: int, parents) -> np.ndarray:
    """[Q][L] True where key t is hidden from query j: a drafted token off j's
    branch. The prefix is visible to every query."""
    Q = len(parents)
    pre = seq_len - Q
    out = np.zeros((Q, seq_len), dtype=bool)
    out[:, pre:] = ~tree_ancestry(parents)
    return out


def causal_mask(seq_len: int, pq) -> np.ndarray:
    """[Q][L] True where key t lies after query position p_j (excluded).

    Drafted tokens form a chain: query j sees the cache up to and including its
    own position, never a later draft ("The Architecture of Memory", "Tree
    Attention Verification", the chain being the one-branch tree).
    """
    return np.arange(seq_len)[None, :] > np.asarray(pq)[:, None]


def attend_scores(c, k_rope_raw, q_nope, q_rope, w_uk, scale, base=10000.0,
                  chunk: int = 1024, parents=None) -> np.ndarray:
    """Masked scores s[j][h][t] = scale * (q_j,h . K_t,h); -inf where t > p_j.

    With ``parents`` (the drafted tree, [Q] ints) the positions and the mask
    are the tree's: tree_positions and tree_excluded.
    """
    c = np.asarray(c, F64)
    L = c.shape[0]
    q_nope = np.asarray(q_nope, F64)
    Q, H, _ = q_nope.shape
    if parents is None:
        pq = query_positions(L, Q)
        kpos = np.arange(L)
        masked = causal_mask(L, pq)                                      # [Q][L]
    else:
        kpos, pq = tree_positions(L, parents)
        masked = tree_excluded(L, parents)
    q = np.concatenate([q_nope, rope(q_rope, pq[:, None], base)], axis=-1)  # [Q][H][dk]
    qh = np.ascontiguousarray(q.transpose(1, 0, 2))                      # [H][Q][dk]
    s = np.empty((H, Q, L), F64)
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        k, _ = expand_kv(c[t0:t1], k_rope_raw[t0:t1], kpos[t0:t1], w_uk, None, base)
        s[:, :, t0:t1] = np.matmul(qh, np.ascontiguousarray(k.transpose(1, 2, 0)))
    s *= scale
    s = s.transpose(1, 0, 2).copy()                                      # [Q][H][L]
    s[np.broadcast_to(masked[:, None, :], s.shape)] = -np.inf
    return s


def attend_sequence(c, k_rope_raw, q_nope, q_rope, w_uk, w_uv, scale,
                    base: float = 10000.0, chunk: int = 1024, parents=None, keep=None):
    """Decode attention of one sequence, without absorption.

    c [L][d_c], k_rope_raw [L][d_r] (unrotated, positions 0..L-1),
    q_nope [Q][H][d_n], q_rope [Q][H][d_r] (unrotated), w_uk [H][d_n][d_c],
    w_uv [H][d_v][d_c]. Textbook softmax: m = max s, p = e^(s-m) / sum e^(s-m).
    Returns o [Q][H][d_v] = sum_t p_t V_t,h, o_lat [Q][H][d_c] = sum_t p_t c_t
    (the same weights applied to the latents) and lse [Q][H] = m + ln sum e^(s-m).
    ``parents``: the drafted tokens form this tree instead of a chain.
    ``keep``: [Q][L] bool, the cached tokens each query reads (a sparse read);
    every kept token must be visible to its query, and the others are left
    out of the softmax.
    """
    c = np.asarray(c, F64)
    L = c.shape[0]
    s = attend_scores(c, k_rope_raw, q_nope, q_rope, w_uk, scale, base, chunk, parents=parents)
    if keep is not None:
        keep = np.asarray(keep, dtype=bool)
        assert keep.shape == (s.shape[0], L)
        if np.any(keep[:, None, :] & np.isneginf(s)):
            raise ValueError("a kept token lies after its query")
        s[np.broadcast_to(~keep[:, None, :], s.shape)] = -np.inf
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=-1, keepdims=True)
    p = e / den
    lse = m[..., 0] + np.log(den[..., 0])
    Q, H = p.shape[:2]
    w_uv = np.asarray(w_uv, F64)
    dv = w_uv.shape[1]
    o = np.zeros((Q, H, dv), F64)
    o_lat = np.zeros((Q, H, c.shape[1]), F64)
    ph = p.transpose(1, 0, 2)                                            # [H][Q][L]
    for t0 in range(0, L, chunk):
        t1 = min(L, t0 + chunk)
        cc = c[t0:t1]
        _, v = expand_kv(cc, None, None, None, w_uv, base)
        o += np.matmul(ph[:, :, t0:t1], np.ascontiguousarray(v.transpose(1, 0, 2))).transpose(1, 0, 2)
        o_lat += np.einsum("qht,tc->qhc", p[:, :, t0:t1], cc, optimize=True)
    return o, o_lat, lse


def mla_decode_ref(inputs, heads: Optional[Sequence[int]] = None,
                   seqs: Optional[Sequence[int]] = None, chunk: int = 1024):
    """Oracle over a whole batch drawn by ``workload.make``.

    Returns dict(o [B][Q][H'][d_v], o_lat [B][Q][H'][d_c], lse [B][Q][H']) for
    the selected heads (all by default) and sequences (all by default; rows of
    unselected sequences are NaN). A workload with a drafted tree
    (``inputs.parents``) is verified under that tree.
    """
    wl = inputs.wl
    hs = list(range(wl.heads)) if heads is None else list(heads)
    bs = list(range(wl.batch)) if seqs is None else list(seqs)
    B, Q = wl.batch, wl.q_len
    o = np.full((B, Q, len(hs), wl.v_dim), np.nan)
    o_lat = np.full((B, Q, len(hs), wl.kv_rank), np.nan)
    lse = np.full((B, Q, len(hs)), np.nan)
    w_uk = np.asarray(inputs.w_uk, F64)[hs]
    w_uv = np.asarray(inputs.w_uv, F64)[hs]
    for b in bs:
        c, kr = inputs.seq(b)
        par = None if getattr(inputs, "parents", None) is None else inputs.parents[b]
        ob, olb, lb = attend_sequence(c, kr, inputs.q_nope[b][:, hs], inputs.q_rope[b][:, hs],
                                      w_uk, w_uv, wl.softmax_scale, wl.rope_base, chunk,
                                      parents=par)
        o[b], o_lat[b], lse[b] = ob, olb, lb
    return {"o": o, "o_lat": o_lat, "lse": lse}


# --------------------------------------------------------------------------
# absorbed algebra (test-only: pins associativity, checks query absorption)
# --------------------------------------------------------------------------
def absorbed_query(q_nope, q_rope, w_uk, pos, base: float = 10000.0) -> np.ndarray:
    """q_full = [W_UK[h]^T q_nope ; RoPE(q_rope, pos)] per (token, head).

    The weight-absorption rearrangement: the content score against the
    expanded key equals the absorbed query against the latent ("The
    Architecture of Memory", "The Weight Absorption Trick"; "DeepSeek's Config
    Says 16 KV Heads", section 5). q_nope [..][H][d_n], q_rope [..][H][d_r],
    w_uk [H][d_n][d_c], pos broadcasting against q_nope.shape[:-2].
    Returns [..][H][d_c + d_r].
    """
    q_nope = np.asarray(q_nope, F64)
    w_uk = np.asarray(w_uk, F64)
    q_lat = np.einsum("...hn,hnc->...hc", q_nope, w_uk)
    pos = np.asarray(pos, F64)[..., None]
    q_pe = rope(q_rope, pos, base)
    return np.concatenate([q_lat, q_pe], axis=-1)


def absorbed_attend_sequence(c, k_rope_raw, q_nope, q_rope, w_uk, w_uv, scale,
                             base: float = 10000.0, parents=None):
    """The same attention scored in latent space and up-projected at the end.

    s = scale * (q_lat . c_t + q_pe . RoPE(k^R_t, t)), o = W_UV (sum_t p_t c_t).
    Used only to pin ``attend_sequence`` (associativity of the products).
    """
    c = np.asarray(c, F64)
    L = c.shape[0]
    Q = np.asarray(q_nope).shape[0]
    if parents is None:
        pq, kpos = query_positions(L, Q), np.arange(L)
        masked = causal_mask(L, pq)
    else:
        kpos, pq = tree_positions(L, parents)
        masked = tree_excluded(L, parents)
    qf = absorbed_query(q_nope, q_rope, w_uk, pq, base)                     # [Q][H][D]
    kf = np.concatenate([c, rope(k_rope_raw, kpos, base)], axis=-1)         # [L][D]
    s = scale * np.einsum("qhd,td->qht", qf, kf)
    s[np.broadcast_to(masked[:, None, :], s.shape)] = -np.inf
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(-1, keepdims=True)
    p = e / den
    o_lat = np.einsum("qht,tc->qhc", p, c)
    o = np.einsum("hvc,qhc->qhv", np.asarray(w_uv, F64), o_lat)
    return o, o_lat, m[..., 0] + np.log(den[..., 0])


# --------------------------------------------------------------------------
# split-KV partials and the log-sum-exp merge
# --------------------------------------------------------------------------
def split_bounds(seq_len: int, num_splits: int, page: int = 64,
                 chunk_tokens: int = 0) -> List[Tuple[int, int]]:
    """Token ranges of the split-KV units of one sequence.

    Reading of "splits the cache into chunks" ("The Architecture of Memory",
    "Flash-Decoding and FlashInfer"): chunk = page * ceil(ceil(L / S) / page)
    tokens, unit s covers [s*chunk, min(L, (s+1)*chunk)); units past the end
    are empty. Chunks are whole pages so a unit never splits a page. With
    chunk_tokens > 0 the chunk is that fixed size for every sequence instead
    (a long sequence then fills more of its S units than a short one).
    """
    if chunk_tokens > 0:
        chunk = chunk_tokens
    else:
        per = -(-seq_len // num_splits)
        chunk = page * (-(-per // page))
    return [(min(seq_len, s * chunk), min(seq_len, (s + 1) * chunk)) for s in range(num_splits)]


def attend_partials(c, k_rope_raw, q_nope, q_rope, w_uk, scale, num_splits,
                    base: float = 10000.0, page: int = 64, chunk_tokens: int = 0,
                    parents=None):
    """Per-split normalised partials of the latent output.

    For unit s over tokens [a, e): o_s = sum_t e^(s_t - m_s) c_t / sum_t e^(s_t - m_s)
    and lse_s = m_s + ln sum_t e^(s_t - m_s), with the same causal mask as the
    full decode. An empty (or fully masked) unit gives o_s = 0, lse_s = -inf.
    Returns o_part [Q][H][S][d_c], lse_part [Q][H][S].
    """
    c = np.asarray(c, F64)
    L = c.shape[0]
    s = attend_scores(c, k_rope_raw, q_nope, q_rope, w_uk, scale, base,
                      parents=parents)                                   # [Q][H][L]
    Q, H = s.shape[:2]
    o_part = np.zeros((Q, H, num_splits, c.shape[1]), F64)
    lse_part = np.full((Q, H, num_splits), -np.inf, F64)
    for si, (a, e) in enumerate(split_bounds(L, num_splits, page, chunk_tokens)):
        if e <= a:
            continue
        ss = s[:, :, a:e]
        m = ss.max(-1, keepdims=True)
        ok = np.isfinite(m[..., 0])
        msafe = np.where(np.isfinite(m), m, 0.0)
        w = np.exp(ss - msafe)
        den = w.sum(-1, keepdims=True)
        o = np.einsum("qht,tc->qhc", w, c[a:e]) / np.where(den > 0, den, 1.0)
        o_part[:, :, si] = np.where(ok[..., None], o, 0.0)
        lse_part[:, :, si] = np.where(ok, msafe[..., 0] + np.log(np.where(den[..., 0] > 0, den[..., 0], 1.0)), -np.inf)
    return o_part, lse_part


def lse_combine(o_part, lse_part):
    """Merge split partials: LSE = ln sum_s e^(lse_s), o = sum_s e^(lse_s - LSE) o_s.

    The log-sum-exp reduction across splits ("The Architecture of Memory",
    "Flash-Decoding and FlashInfer"). o_part [..][S][d], lse_part [..][S].
    Splits with lse = -inf contribute nothing.
    """
    o_part = np.asarray(o_part, F64)
    lse_part = np.asarray(lse_part, F64)
    m = lse_part.max(axis=-1, keepdims=True)
    w = np.exp(lse_part - m)
    tot = w.sum(axis=-1, keepdims=True)
    lse = (m + np.log(tot))[..., 0]
    o = np.einsum("...s,...sd->...d", w / tot, o_part)
    return o, lse


# --------------------------------------------------------------------------
# 8-bit latent cache
# --------------------------------------------------------------------------
Q8_LEVELS = 255  # codes 0 .. 255


def quantize_q8(x):
    """Asymmetric 8-bit codes of one row part between its min and max.

    The row's minimum and maximum fix the range; the step is (max - min) /
    255; a value's code is its distance from the minimum in steps, rounded to
    the nearest integer (ties to even). All in float32, the precision the
    codes are decided in. A constant part (max == min) has step 0 and codes 0.
    Returns (codes uint8 [n], minimum float32, step float32).
    """
    x = np.asarray(x, dtype=np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(Q8_LEVELS))
    if step == 0:
        return np.zeros(x.shape, dtype=np.uint8), mn, step
    codes = np.rint((x - mn) / step)
    return np.clip(codes, 0, Q8_LEVELS).astype(np.uint8), mn, step


def dequantize_q8(codes, mn, step):
    """The value a code stands for: min + code * step (float64)."""
    return F64(mn) + np.asarray(codes, F64) * F64(step)


# --------------------------------------------------------------------------
# 4-bit latent cache: the same per-row coding with 16 levels
# ("KV Cache Optimization: Scaling to Million-Token Contexts", technique 3,
# whose listing defaults to 4 bits, and its comparison table: INT4, 4x)
# --------------------------------------------------------------------------
Q4_LEVELS = 15  # codes 0 .. 15


def quantize_q4(x):
    """Asymmetric 4-bit codes of one row part between its min and max: step =
    (max - min) / 15, code = the distance from the minimum in steps rounded to
    the nearest integer (ties to even), in float32; a constant part has step
    0 and codes 0. Returns (codes uint8 [n] in 0 .. 15, minimum, step)."""
    x = np.asarray(x, dtype=np.float32)
    mn, mx = np.float32(x.min()), np.float32(x.max())
    step = np.float32((mx - mn) / np.float32(Q4_LEVELS))
    if step == 0:
        return np.zeros(x.shape, dtype=np.uint8), mn, step
    codes = np.rint((x - mn) / step)
    return np.clip(codes, 0, Q4_LEVELS).astype(np.uint8), mn, step


def pack_q4(codes):
    """Two 4-bit codes per byte: column 2i in the low nibble of byte i and
    column 2i + 1 in its high nibble (the layout of a 4-bit cache row)."""
    codes = np.asarray(codes, np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_q4(packed):
    """Inverse of pack_q4: the 4-bit codes of each byte, low nibble first."""
    packed = np.asarray(packed, np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out


def quantize_cache_rows(c, k_rope_rotated_f32, bits: int = 8):
    """Quantize cached rows [c ; k^R] per token in ``bits`` (8 or 4) bits, the
    latent part and the RoPE part each on its own range. Inputs float32
    [T][d_c], [T][d_r] (the RoPE keys already rotated and in float32). Returns
    dict(codes uint8 [T][D] (one code per entry, unpacked), lat_min, lat_step,
    rope_min, rope_step float32 [T]) and the dequantized rows float64
    (c_hat [T][d_c], k_hat [T][d_r])."""
    quant = {8: quantize_q8, 4: quantize_q4}[bits]
    c = np.asarray(c, np.float32)
    k = np.asarray(k_rope_rotated_f32, np.float32)
    T, dc = c.shape
    dr = k.shape[1]
    codes = np.empty((T, dc + dr), np.uint8)
    meta = {n: np.empty(T, np.float32) for n in ("lat_min", "lat_step", "rope_min", "rope_step")}
    c_hat = np.empty((T, dc), F64)
    k_hat = np.empty((T, dr), F64)
    for t in range(T):
        q, mn, st = quant(c[t])
        codes[t, :dc], meta["lat_min"][t], meta["lat_step"][t] = q, mn, st
        c_hat[t] = dequantize_q8(q, mn, st)
        q, mn, st = quant(k[t])
        codes[t, dc:], meta["rope_min"][t], meta["rope_step"][t] = q, mn, st
        k_hat[t] = dequantize_q8(q, mn, st)
    return dict(codes=codes, **meta), c_hat, k_hat


def rotated_keys_f32(k_rope_raw, positions, base: float = 10000.0) -> np.ndarray:
    """RoPE keys rotated at their positions in float64, then rounded to float32
    (the values an 8-bit cache row quantizes)."""
    return rope(k_rope_raw, positions, base).astype(np.float32)


def attend_sequence_rotated(c, k_rotated, q_nope, q_rope, w_uk, w_uv, scale,
                            base: float = 10000.0, parents=None):
    """attend_sequence over a cache whose RoPE keys are given already rotated
    (as an 8-bit cache stores them): the same unabsorbed attention, the key
    positions entering only through the stored rotation."""
    c = np.asarray(c, F64)
    k_rotated = np.asarray(k_rotated, F64)
    L = c.shape[0]
    q_nope = np.asarray(q_nope, F64)
    Q, H, _ = q_nope.shape
    if parents is None:
        pq = query_positions(L, Q)
        masked = causal_mask(L, pq)
    else:
        _, pq = tree_positions(L, parents)
        masked = tree_excluded(L, parents)
    q = np.concatenate([q_nope, rope(q_rope, pq[:, None], base)], axis=-1)   # [Q][H][dk]
    w_uk = np.asarray(w_uk, F64)
    Hk, dn, dc = w_uk.shape
    kc = (c @ w_uk.reshape(Hk * dn, dc).T).reshape(L, Hk, dn)
    k = np.concatenate([kc, np.broadcast_to(k_rotated[:, None, :], (L, Hk, k_rotated.shape[1]))],
                       axis=-1)                                               # [L][H][dk]
    s = scale * np.einsum("qhd,thd->qht", q, k)
    s[np.broadcast_to(masked[:, None, :], s.shape)] = -np.inf
    m = s.max(-1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(-1, keepdims=True)
    p = e / den
    w_uv = np.asarray(w_uv, F64)
    v = (c @ w_uv.reshape(-1, dc).T).reshape(L, w_uv.shape[0], w_uv.shape[1])
    o = np.einsum("qht,thv->qhv", p, v)
    o_lat = np.einsum("qht,tc->qhc", p, c)
    return o, o_lat, m[..., 0] + np.log(den[..., 0])


def mla_decode_ref_q8(inputs, heads: Optional[Sequence[int]] = None,
                      seqs: Optional[Sequence[int]] = None, bits: int = 8):
    """The oracle over an 8-bit (or, with bits=4, 4-bit) latent cache: every
    cached row of ``inputs`` is quantized as the cache stores it
    (quantize_cache_rows, RoPE keys rotated at their positions first) and the
    decode attends over the dequantized rows. Returns the dict of
    mla_decode_ref plus "rows" (codes and ranges) per selected sequence for
    the append checks."""
    wl = inputs.wl
    hs = list(range(wl.heads)) if heads is None else list(heads)
    bs = list(range(wl.batch)) if seqs is None else list(seqs)
    B, Q = wl.batch, wl.q_len
    o = np.full((B, Q, len(hs), wl.v_dim), np.nan)
    o_lat = np.full((B, Q, len(hs), wl.kv_rank), np.nan)
    lse = np.full((B, Q, len(hs)), np.nan)
    w_uk = np.asarray(inputs.w_uk, F64)[hs]
    w_uv = np.asarray(inputs.w_uv, F64)[hs]
    rows = {}
    for b in bs:
        c, kr = inputs.seq(b)
        L = c.shape[0]
        par = None if getattr(inputs, "parents", None) is None else inputs.parents[b]
        kpos = np.arange(L) if par is None else tree_positions(L, par)[0]
        qrows, c_hat, k_hat = quantize_cache_rows(c, rotated_keys_f32(kr, kpos, wl.rope_base),
                                                  bits)
        rows[b] = qrows
        o[b], o_lat[b], lse[b] = attend_sequence_rotated(
            c_hat, k_hat, inputs.q_nope[b][:, hs], inputs.q_rope[b][:, hs], w_uk, w_uv,
            wl.softmax_scale, wl.rope_base, parents=par)
    return {"o": o, "o_lat": o_lat, "lse": lse, "rows": rows}


def mla_decode_ref_q4(inputs, heads: Optional[Sequence[int]] = None,
                      seqs: Optional[Sequence[int]] = None):
    """The oracle over a 4-bit latent cache (mla_decode_ref_q8 with 16 levels)."""
    return mla_decode_ref_q8(inputs, heads=heads, seqs=seqs, bits=4)


# --------------------------------------------------------------------------
# chunked prefill: the prompt enters the cache chunk by chunk
# --------------------------------------------------------------------------
def prefill_in_chunks(c, k_rope_raw, q_nope, q_rope, w_uk, w_uv, scale, chunk: int,
                      base: float = 10000.0, cached: int = 0):
    """Prefill of a prompt in chunks of ``chunk`` tokens ("Beyond the Attention
    Bottleneck", "Chunked Prefilling": the prompt is split into chunks that
    are processed one after another, each adding its tokens to the cache).

    c [N][d_c], k_rope_raw [N][d_r]: every token of the sequence, the first
    ``cached`` already in the cache; q_nope [N - cached][H][d_n], q_rope
    [N - cached][H][d_r]: the queries of the prompt tokens that are still to
    be prefilled. Chunk by chunk, tokens [s, e) join the cache and their
    queries attend to the cache as it then stands (tokens 0 .. e-1), query i
    at position s + i seeing t <= s + i. Returns (o, o_lat, lse) for the
    prompt's queries in order.
    """
    N = len(c)
    outs = []
    for s in range(cached, N, chunk):
        e = min(N, s + chunk)
        outs.append(attend_sequence(c[:e], k_rope_raw[:e], q_nope[s - cached:e - cached],
                                    q_rope[s - cached:e - cached], w_uk, w_uv, scale, base))
    return tuple(np.concatenate([o[i] for o in outs]) for i in range(3))


# --------------------------------------------------------------------------
# sparse read: a small scorer picks the cached tokens attention reads
# --------------------------------------------------------------------------
def indexer_scores(q_idx, w_idx, k_idx) -> np.ndarray:
    """Index scores [Q][L] that rate every cached token for each query token.

    The pages fix the scorer's size (64 heads of 128 dimensions) and its role:
    it rates all earlier tokens and attention then reads only the best ones
    ("DeepSeek's Config Says 16 KV Heads, Its Cache Holds a Ninth of That",
    section 6, "Sparse attention"). Reading (the DSA published form, the pages
    print no formula): I[j][t] = sum_h w[j][h] * max(0, q[j][h] . k[t]), with
    q_idx [Q][H_I][d_I], per-query head weights w_idx [Q][H_I] and one indexer
    key per cached token, k_idx [L][d_I].
    """
    q = np.asarray(q_idx, F64)
    w = np.asarray(w_idx, F64)
    k = np.asarray(k_idx, F64)
    dots = np.matmul(q, k.T)                                      # [Q][H_I][L]
    return np.einsum("qh,qht->qt", w, np.maximum(dots, 0.0))


def topk_tokens(scores, k: int, visible: int) -> np.ndarray:
    """Cached tokens one query reads: of tokens 0 .. visible-1, the k with the
    highest index scores (every one when visible <= k), in increasing token
    order (same page and section: attention runs only over the top 2,048).
    Reading: equal scores go to the smaller token index; NaN among the
    visible scores makes the selection undefined (ValueError)."""
    s = np.asarray(scores, F64)[:visible]
    if np.isnan(s).any():
        raise ValueError("NaN index score")
    if visible <= k:
        return np.arange(visible)
    order = np.lexsort((np.arange(visible), -s))                  # score desc, index asc
    return np.sort(order[:k])


def dsa_selection(inputs) -> List[List[np.ndarray]]:
    """[B][Q] selected token arrays of a workload with a sparse read: indexer
    scores of every cached token, then the top index_topk among those query j
    sees (t <= L - Q + j)."""
    wl = inputs.wl
    out = []
    for b in range(wl.batch):
        L = int(inputs.seq_lens[b])
        sc = indexer_scores(inputs.q_idx[b], inputs.w_idx[b], inputs.seq_index_keys(b))
        out.append([topk_tokens(sc[j], wl.index_topk, L - wl.q_len + j + 1)
                    for j in range(wl.q_len)])
    return out


def mla_decode_ref_sparse(inputs, selection=None, heads: Optional[Sequence[int]] = None,
                          seqs: Optional[Sequence[int]] = None):
    """The oracle of a sparse read: query j of sequence b attends only over the
    cached tokens selection[b][j] (dsa_selection by default). Returns the dict
    of mla_decode_ref plus "selection"."""
    wl = inputs.wl
    sel = dsa_selection(inputs) if selection is None else selection
    hs = list(range(wl.heads)) if heads is None else list(heads)
    bs = list(range(wl.batch)) if seqs is None else list(seqs)
    B, Q = wl.batch, wl.q_len
    o = np.full((B, Q, len(hs), wl.v_dim), np.nan)
    o_lat = np.full((B, Q, len(hs), wl.kv_rank), np.nan)
    lse = np.full((B, Q, len(hs)), np.nan)
    w_uk = np.asarray(inputs.w_uk, F64)[hs]
    w_uv = np.asarray(inputs.w_uv, F64)[hs]
    for b in bs:
        c, kr = inputs.seq(b)
        L = c.shape[0]
        keep = np.zeros((Q, L), dtype=bool)
        for j in range(Q):
            keep[j, np.asarray(sel[b][j], dtype=np.int64)] = True
        o[b], o_lat[b], lse[b] = attend_sequence(c, kr, inputs.q_nope[b][:, hs],
                                                 inputs.q_rope[b][:, hs], w_uk, w_uv,
                                                 wl.softmax_scale, wl.rope_base, keep=keep)
    return {"o": o, "o_lat": o_lat, "lse": lse, "selection": sel}


# --------------------------------------------------------------------------
# paged cache append (expected pool image)
# --------------------------------------------------------------------------
def cache_slot(page_table, seq: int, pos: int, page: int = 64) -> int:
    """Physical row of logical token ``pos`` of sequence ``seq``:
    page_table[seq][pos // page] * page + pos % page."""
    return int(page_table[seq][pos // page]) * page + pos % page


def cache_append_image(pool, c, k_rope, seq_idx, pos, page_table, kv_rank: int,
                       page: int = 64, rotate: bool = False, base: float = 10000.0,
                       rope_pos=None):
    """The pool after appending rows [c_n ; k^R_n] at (seq_idx[n], pos[n]).

    ``pool`` is [P][page][D] in any dtype and is copied, never modified. Raw
    mode copies the values as given (so a bit pattern array gives a byte-exact
    image); rotate mode stores RoPE(k^R_n, pos[n]) in fp64 instead, the rotated
    positional key the cache carries ("Beyond the Attention Bottleneck", "The
    RoPE Compatibility Problem"). With ``rope_pos`` the key is rotated by
    rope_pos[n] while pos[n] still picks the slot (a drafted tree's token).
    """
    out = np.array(pool, copy=True)
    P, pg, D = out.shape
    assert pg == page
    flat = out.reshape(P * page, D)
    if rotate:
        flat = flat.astype(F64)
    for n in range(len(pos)):
        slot = cache_slot(page_table, int(seq_idx[n]), int(pos[n]), page)
        flat[slot, :kv_rank] = c[n]
        rp = pos[n] if rope_pos is None else rope_pos[n]
        flat[slot, kv_rank:] = rope(k_rope[n], rp, base) if rotate else k_rope[n]
    return flat.reshape(P, page, D)
