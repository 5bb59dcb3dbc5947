"""Seeded synthetic MLA decode workloads.

Shapes follow the model facts the pages give for the MLA family: a 512-wide
latent plus a 64-wide decoupled-RoPE key per token and layer, 16 heads for
DeepSeek-V2-Lite and 128 for DeepSeek-V2/V3 ("DeepSeek's Config Says 16 KV
Heads, Its Cache Holds a Ninth of That", section 5 "Multi-head latent attention
(MLA)"), 64-token pages mapped through a page table ("The Architecture of
Memory", "PagedAttention: Virtual Memory for LLMs"), and a 32,768-token
conversation as the reference context length (same page, introduction).

Value recipe (the pages print no data): latents, RoPE keys and queries are
N(0, 1); W_UK and W_UV are N(0, 1/d_c). Draws are made in float32 and, for bf16
workloads, rounded to the nearest bf16 (ties to even); the returned float32
arrays then hold exactly the values the GPU reads, so the oracle can upcast
them to float64 without a second rounding.

Every tensor has its own counter-free stream, ``default_rng(SeedSequence([seed,
tag, index]))``, so one sequence's latents can be regenerated without drawing
any other tensor. Nothing here computes attention, RoPE or any projection.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

PAGE = 64

# stream tags: one independent generator per tensor (and per sequence)
_T_LENS, _T_WUK, _T_WUV, _T_QN, _T_QR, _T_C, _T_KR, _T_PERM, _T_TREE = range(9)
_T_QI, _T_WI, _T_KI, _T_SEL, _T_SCORES = range(9, 14)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    heads: int
    kv_rank: int          # d_c, latent width
    rope_dim: int         # d_r, decoupled RoPE key width
    nope_dim: int         # d_n, per-head content query/key width
    v_dim: int            # d_v, per-head value width
    dtype: str            # "f32" or "bf16"
    seq_len: Optional[int] = None            # fixed length for every sequence
    len_range: Optional[tuple] = None        # inclusive (lo, hi) uniform lengths
    paged: bool = False   # True: one seeded permutation of the page pool
    num_splits: int = 1   # split-KV partitions per sequence used by the bench
    split_chunk: int = 0  # > 0: every partition holds this many tokens (fixed-size plan)
    page_size: int = PAGE
    rope_base: float = 10000.0
    # drafted tokens (the last q_len of each sequence): None = a chain; a
    # tuple = that parent array for every sequence; "random" = a seeded
    # random tree per sequence (parent of token j uniform in [-1, j-1])
    tree: object = None
    # cache format: "native" = rows in the workload dtype; "q8" = 8-bit codes
    # per row part plus (min, step) pairs, D + 16 bytes per token; "q4" =
    # 4-bit codes, two per byte, plus the same pairs, D / 2 + 16 bytes
    cache: str = "native"
    # sparse read: > 0 = each query reads only the index_topk cached tokens an
    # indexer of index_heads heads x index_dim rates highest
    index_topk: int = 0
    index_heads: int = 64
    index_dim: int = 128
    # True: indexer queries and keys are integers in [-2, 2] and head weights
    # multiples of 1/8 in [-2, 2], so every index score is exact in float32
    # whatever the summation order (both sides then rank identical values)
    index_exact: bool = False
    description: str = ""

    @property
    def dim(self) -> int:
        """Cached row width D = d_c + d_r."""
        return self.kv_rank + self.rope_dim

    @property
    def softmax_scale(self) -> float:
        """1/sqrt(d_n + d_r): the width of one head's full query/key."""
        return 1.0 / math.sqrt(self.nope_dim + self.rope_dim)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def cache_row_bytes(self) -> int:
        """Bytes one cached token occupies (per layer)."""
        if self.cache == "q8":
            return self.dim + 16
        if self.cache == "q4":
            return self.dim // 2 + 16
        return self.dim * self.elem_bytes

    @property
    def max_seq_len(self) -> int:
        return self.seq_len if self.seq_len is not None else int(self.len_range[1])

    @property
    def max_pages(self) -> int:
        return -(-self.max_seq_len // self.page_size)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_f32", batch=1, q_len=1, heads=4, kv_rank=64, rope_dim=16,
                 nope_dim=32, v_dim=32, dtype="f32", seq_len=256, num_splits=4,
                 description="tiny fp32 MLA decode, H=4, d_c=64, d_r=16, L=256"),
        Workload("v2lite_32k", batch=8, q_len=1, heads=16, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, dtype="bf16", seq_len=32768, num_splits=32,
                 description="DeepSeek-V2-Lite layer shape, B=8, L=32768, contiguous"),
        Workload("v2lite_paged_varlen", batch=32, q_len=1, heads=16, kv_rank=512,
                 rope_dim=64, nope_dim=128, v_dim=128, dtype="bf16",
                 len_range=(1024, 32768), paged=True, num_splits=16,
                 description="V2-Lite shape, B=32, L~U[1024,32768], permuted 64-token pages"),
        Workload("v2_h128_8k", batch=64, q_len=1, heads=128, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, dtype="bf16", seq_len=8192, paged=True,
                 num_splits=2,
                 description="DeepSeek-V2 head count, B=64, L=8192, permuted pages"),
        Workload("v2_h128_1m_q4", batch=1, q_len=4, heads=128, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, dtype="bf16", seq_len=1048576, num_splits=256,
                 description="1M-token context, Q=4 chain verify, H=128, contiguous"),
        # tree-structured speculative verification: 8 drafted tokens, a root
        # with two children, each with two children, one of which has a child
        Workload("v2lite_32k_q8", batch=8, q_len=1, heads=16, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, dtype="bf16", seq_len=32768, num_splits=32,
                 cache="q8",
                 description="DeepSeek-V2-Lite layer shape, B=8, L=32768, 8-bit latent cache"),
        Workload("v2lite_32k_q4", batch=8, q_len=1, heads=16, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, dtype="bf16", seq_len=32768, num_splits=32,
                 cache="q4",
                 description="DeepSeek-V2-Lite layer shape, B=8, L=32768, 4-bit latent cache"),
        Workload("v2lite_32k_dsa", batch=8, q_len=1, heads=16, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, dtype="bf16", seq_len=32768, num_splits=16,
                 index_topk=2048,
                 description="V2-Lite shape, B=8, L=32768, sparse read of the top 2,048 tokens "
                             "chosen by a 64-head x 128 indexer"),
        # chunked prefill: the last 4,096-token chunk of a 32,768-token prompt
        # (its queries attend causally to the 28,672 cached tokens and to the
        # chunk itself)
        Workload("v2lite_prefill_32k_c4k", batch=1, q_len=4096, heads=16, kv_rank=512,
                 rope_dim=64, nope_dim=128, v_dim=128, dtype="bf16", seq_len=32768,
                 num_splits=1,
                 description="V2-Lite shape, prefill of the last 4,096-token chunk of a "
                             "32,768-token prompt"),
        Workload("v2lite_32k_tree8", batch=8, q_len=8, heads=16, kv_rank=512, rope_dim=64,
                 nope_dim=128, v_dim=128, dtype="bf16", seq_len=32768, num_splits=16,
                 tree=(-1, 0, 0, 1, 1, 2, 2, 3),
                 description="V2-Lite shape, B=8, L=32768, 8 drafted tokens in a tree, one pass"),
    ]
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 values.

    Finite inputs only (the draws are finite): their bit patterns are at most
    0xFF7FFFFF, so adding 0x8000 cannot wrap a uint32.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).copy()
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _rng(seed: int, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), tag, idx]))


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_bf16(x) if dtype == "bf16" else x


def seq_lengths(wl: Workload, seed: int = 0) -> np.ndarray:
    if wl.seq_len is not None:
        return np.full(wl.batch, wl.seq_len, dtype=np.int32)
    lo, hi = wl.len_range
    return _rng(seed, _T_LENS).integers(lo, hi, endpoint=True, size=wl.batch).astype(np.int32)


def seq_latents(wl: Workload, seed: int, b: int, length: int):
    """(c [length][d_c], k_rope [length][d_r]) of sequence b, unrotated keys."""
    c = _normal(_rng(seed, _T_C, b), (length, wl.kv_rank), 1.0, wl.dtype)
    kr = _normal(_rng(seed, _T_KR, b), (length, wl.rope_dim), 1.0, wl.dtype)
    return c, kr


def _small_ints(rng, shape, lo, hi, scale=1.0):
    return (rng.integers(lo, hi, endpoint=True, size=shape).astype(np.float32)
            * np.float32(scale))


def seq_index_keys(wl: Workload, seed: int, b: int, length: int) -> np.ndarray:
    """Indexer keys [length][d_I] of sequence b: N(0, 1) in the workload dtype,
    or integers in [-2, 2] with ``index_exact``."""
    if wl.index_exact:
        return _small_ints(_rng(seed, _T_KI, b), (length, wl.index_dim), -2, 2)
    return _normal(_rng(seed, _T_KI, b), (length, wl.index_dim), 1.0, wl.dtype)


def random_selection(seed: int, b: int, j: int, visible: int, k: int) -> np.ndarray:
    """A seeded set of min(k, visible) distinct tokens of 0 .. visible-1, in
    increasing order: an index list for a sparse read drawn without any
    scores (for testing the sparse decode on its own)."""
    rng = _rng(seed, _T_SEL, b * 4096 + j)
    if visible <= k:
        return np.arange(visible, dtype=np.int32)
    return np.sort(rng.choice(visible, size=k, replace=False)).astype(np.int32)


def score_rows(seed: int, rows: int, length: int, ties: bool = True) -> np.ndarray:
    """float32 [rows][length] index scores for testing top-k selection alone:
    N(0, 4) values, and with ``ties`` a quarter of them copied from a few
    shared values (exact ties, +0.0 and -0.0 among them) so that the tie rule
    decides the boundary."""
    rng = _rng(seed, _T_SCORES, rows * 65536 + length)
    x = rng.standard_normal(size=(rows, length), dtype=np.float32) * np.float32(2.0)
    if ties:
        shared = np.array([0.0, -0.0, 1.5, 2.25, 3.0, -1.0], dtype=np.float32)
        pick = rng.random((rows, length)) < 0.25
        x[pick] = shared[rng.integers(0, len(shared), size=int(pick.sum()))]
    return x


def tree_parents(wl: Workload, seed: int = 0) -> Optional[np.ndarray]:
    """[B][Q] int32 parent of each drafted token (-1: attached to the prefix),
    or None for a chain. Parents always precede their children."""
    if wl.tree is None:
        return None
    Q = wl.q_len
    if wl.tree == "random":
        out = np.empty((wl.batch, Q), dtype=np.int32)
        for b in range(wl.batch):
            rng = _rng(seed, _T_TREE, b)
            out[b] = [-1] + [int(rng.integers(-1, j, endpoint=False)) for j in range(1, Q)]
        return out
    par = np.asarray(wl.tree, dtype=np.int32)
    assert par.shape == (Q,) and all(-1 <= int(p) < j for j, p in enumerate(par))
    return np.broadcast_to(par, (wl.batch, Q)).copy()


def page_table_for(wl: Workload, seq_lens: np.ndarray, seed: int = 0):
    """Logical->physical page map [B][max_pages] (-1 = unused) and pool size.

    The pool holds exactly sum(ceil(L_b / page)) pages. Pages are handed out in
    sequence order; with ``paged`` they come from one seeded permutation of the
    pool, otherwise each sequence owns a contiguous run (identity layout).
    """
    npg = [-(-int(L) // wl.page_size) for L in seq_lens]
    total = int(sum(npg))
    order = (_rng(seed, _T_PERM).permutation(total) if wl.paged
             else np.arange(total))
    pt = np.full((wl.batch, wl.max_pages), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(npg):
        pt[b, :n] = order[k:k + n]
        k += n
    return pt, total


@dataclasses.dataclass
class Inputs:
    wl: Workload
    seed: int
    seq_lens: np.ndarray          # int32 [B]
    offsets: np.ndarray           # int64 [B+1], token offsets into c / k_rope
    w_uk: np.ndarray              # [H][d_n][d_c]
    w_uv: np.ndarray              # [H][d_v][d_c]
    q_nope: np.ndarray            # [B][Q][H][d_n]
    q_rope: np.ndarray            # [B][Q][H][d_r], unrotated
    page_table: np.ndarray        # int32 [B][max_pages]
    num_pages: int
    c: Optional[np.ndarray] = None        # [sum L_b][d_c]
    k_rope: Optional[np.ndarray] = None   # [sum L_b][d_r], unrotated
    parents: Optional[np.ndarray] = None  # int32 [B][Q] drafted tree (None: chain)
    q_idx: Optional[np.ndarray] = None    # [B][Q][H_I][d_I] indexer queries
    w_idx: Optional[np.ndarray] = None    # float32 [B][Q][H_I] indexer head weights
    k_idx: Optional[np.ndarray] = None    # [sum L_b][d_I] indexer keys

    def seq(self, b: int):
        """Latents and unrotated RoPE keys of sequence b (views or fresh draws)."""
        if self.c is not None:
            s, e = int(self.offsets[b]), int(self.offsets[b + 1])
            return self.c[s:e], self.k_rope[s:e]
        return seq_latents(self.wl, self.seed, b, int(self.seq_lens[b]))

    def seq_index_keys(self, b: int) -> np.ndarray:
        """Indexer keys [L_b][d_I] of sequence b."""
        if self.k_idx is not None:
            return self.k_idx[int(self.offsets[b]):int(self.offsets[b + 1])]
        return seq_index_keys(self.wl, self.seed, b, int(self.seq_lens[b]))


def make(wl: Workload, seed: int = 0, with_latents: bool = True,
         seq_lens: Optional[Sequence[int]] = None) -> Inputs:
    """Draw every input of one decode step of ``wl``.

    ``seq_lens`` overrides the drawn lengths (used for edge cases); latents are
    still drawn per sequence from the same streams.
    """
    lens = (np.asarray(seq_lens, dtype=np.int32) if seq_lens is not None
            else seq_lengths(wl, seed))
    assert lens.shape == (wl.batch,)
    H, dn, dv, dc, dr = wl.heads, wl.nope_dim, wl.v_dim, wl.kv_rank, wl.rope_dim
    wstd = 1.0 / math.sqrt(dc)
    w_uk = _normal(_rng(seed, _T_WUK), (H, dn, dc), wstd, wl.dtype)
    w_uv = _normal(_rng(seed, _T_WUV), (H, dv, dc), wstd, wl.dtype)
    q_nope = _normal(_rng(seed, _T_QN), (wl.batch, wl.q_len, H, dn), 1.0, wl.dtype)
    q_rope = _normal(_rng(seed, _T_QR), (wl.batch, wl.q_len, H, dr), 1.0, wl.dtype)
    offsets = np.zeros(wl.batch + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens.astype(np.int64))
    pt, total = page_table_for(wl, lens, seed)
    inp = Inputs(wl, seed, lens, offsets, w_uk, w_uv, q_nope, q_rope, pt, total,
                 parents=tree_parents(wl, seed))
    if wl.index_topk > 0:
        Hi, di = wl.index_heads, wl.index_dim
        if wl.index_exact:
            inp.q_idx = _small_ints(_rng(seed, _T_QI), (wl.batch, wl.q_len, Hi, di), -2, 2)
            inp.w_idx = _small_ints(_rng(seed, _T_WI), (wl.batch, wl.q_len, Hi), -16, 16, 0.125)
        else:
            inp.q_idx = _normal(_rng(seed, _T_QI), (wl.batch, wl.q_len, Hi, di), 1.0, wl.dtype)
            inp.w_idx = _normal(_rng(seed, _T_WI), (wl.batch, wl.q_len, Hi), 1.0 / math.sqrt(Hi),
                                "f32")
    if with_latents:
        T = int(offsets[-1])
        fdt = np.float32
        inp.c = np.empty((T, dc), dtype=fdt)
        inp.k_rope = np.empty((T, dr), dtype=fdt)
        for b in range(wl.batch):
            c, kr = seq_latents(wl, seed, b, int(lens[b]))
            inp.c[offsets[b]:offsets[b + 1]] = c
            inp.k_rope[offsets[b]:offsets[b + 1]] = kr
        if wl.index_topk > 0:
            inp.k_idx = np.empty((T, wl.index_dim), dtype=fdt)
            for b in range(wl.batch):
                inp.k_idx[offsets[b]:offsets[b + 1]] = seq_index_keys(wl, seed, b, int(lens[b]))
    return inp
