"""ctypes binding of include/mla.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

F32, BF16 = 0, 1
APPEND_RAW, APPEND_ROTATE = 0, 1
_STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE",
           4: "MLA_ERR_ALIGN", 5: "MLA_ERR_CAPACITY", 6: "MLA_ERR_UNSUPPORTED", 7: "MLA_ERR_HIP"}


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


class _Cfg(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("kv_rank", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32), ("nope_dim", ctypes.c_int32),
                ("v_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("rope_base", ctypes.c_float)]


@dataclasses.dataclass(frozen=True)
class Config:
    """Mirror of mla_config_t. ``softmax_scale`` defaults to 1/sqrt(d_n + d_r)."""
    num_heads: int
    kv_rank: int = 512
    rope_dim: int = 64
    nope_dim: int = 128
    v_dim: int = 128
    page_size: int = 64
    dtype: int = BF16
    softmax_scale: Optional[float] = None
    rope_base: float = 10000.0

    @property
    def dim(self) -> int:
        return self.kv_rank + self.rope_dim

    @property
    def scale(self) -> float:
        return (self.softmax_scale if self.softmax_scale is not None
                else 1.0 / math.sqrt(self.nope_dim + self.rope_dim))

    def c(self) -> _Cfg:
        return _Cfg(self.num_heads, self.kv_rank, self.rope_dim, self.nope_dim, self.v_dim,
                    self.page_size, self.dtype, self.scale, self.rope_base)

    def cptr(self):
        """A pointer to this config's mla_config_t, built once per Config (the
        struct is never written)."""
        p = _CPTR.get(self)
        if p is None:
            p = _CPTR[self] = ctypes.pointer(self.c())
        return p

    @staticmethod
    def from_workload(wl) -> "Config":
        return Config(num_heads=wl.heads, kv_rank=wl.kv_rank, rope_dim=wl.rope_dim,
                      nope_dim=wl.nope_dim, v_dim=wl.v_dim, page_size=wl.page_size,
                      dtype=F32 if wl.dtype == "f32" else BF16,
                      softmax_scale=wl.softmax_scale, rope_base=wl.rope_base)


_lib = None
_CPTR = {}  # Config -> pointer to its mla_config_t


def lib_path() -> str:
    return LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libmla.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmla.so not found at {LIB_PATH}: build it first "
                           "(python -m mla_latent_kv_03_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, VP, FP = (ctypes.POINTER(_Cfg), ctypes.c_int32, ctypes.c_int64,
                           ctypes.c_void_p, ctypes.c_void_p)
    sig = {
        "mla_build_info": (ctypes.c_char_p, []),
        "mla_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "mla_config_validate": (ctypes.c_int, [P]),
        "mla_cache_bytes_per_token": (ctypes.c_size_t, [P]),
        "mla_split_chunk": (ctypes.c_int, [P, I32, I32, ctypes.POINTER(ctypes.c_int32)]),
        "mla_default_num_splits": (ctypes.c_int32, [P, I32, I32, I32, I32]),
        "mla_decode_partials_bytes": (ctypes.c_size_t, [P, I32, I32, I32]),
        "mla_decode_kernel_name": (ctypes.c_char_p, [P, I32]),
        "mla_absorb_q": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, VP]),
        "mla_cache_append": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, I32, I32, VP, I64, I32, VP]),
        "mla_decode_paged": (ctypes.c_int, [P, I32, I32, I32, I32, VP, VP, I64, VP, I32, VP, FP, FP, VP]),
        "mla_splitkv_combine": (ctypes.c_int, [P, I32, I32, I32, FP, FP, VP, FP, VP]),
        "mla_up_project_v": (ctypes.c_int, [P, I32, VP, VP, VP, VP]),
        "mla_absorb_append": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, I32, VP, VP, VP, VP, VP,
                                             I32, I32, VP, I64, I32, VP]),
        "mla_combine_up_project": (ctypes.c_int, [P, I32, I32, I32, FP, FP, VP, FP, VP, VP, VP]),
        "mla_decode_paged_chunked": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, VP, I64, VP, I32,
                                                    VP, FP, FP, VP]),
        "mla_chunk_plan": (ctypes.c_int, [P, I64, I32, I32, ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ctypes.c_int32)]),
        "mla_cache_append_at": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, VP, I32, I32, VP, I64,
                                               I32, VP]),
        "mla_absorb_append_at": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, I32, VP, VP, VP, VP,
                                                VP, VP, I32, I32, VP, I64, I32, VP]),
        "mla_decode_paged_tree": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, VP, I64, VP, I32,
                                                 VP, VP, FP, FP, VP]),
        "mla_cache_q8_bytes_per_token": (ctypes.c_size_t, [P]),
        "mla_cache_q4_bytes_per_token": (ctypes.c_size_t, [P]),
        "mla_cache_append_q4": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, VP, I32, I32, VP, I64,
                                               I32, VP]),
        "mla_decode_paged_q4": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, VP, I64, VP, I32,
                                               VP, VP, FP, FP, VP]),
        "mla_cache_append_q8": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, VP, I32, I32, VP, I64,
                                               I32, VP]),
        "mla_decode_paged_q8": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, VP, I64, VP, I32,
                                               VP, VP, FP, FP, VP]),
        "mla_index_append": (ctypes.c_int, [P, I32, I32, VP, VP, VP, VP, I32, I32, VP, I64, VP]),
        "mla_index_scores": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, FP, VP, I64, VP, I32,
                                            VP, FP, I32, VP]),
        "mla_topk_select": (ctypes.c_int, [I32, I32, I32, I32, FP, I32, VP, VP, VP, VP, VP]),
        "mla_index_scores_topk": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, FP, VP, I64, VP,
                                                 I32, VP, FP, I32, I32, VP, VP, VP, VP]),
        "mla_topk_workspace_bytes": (ctypes.c_size_t, [I32, I32]),
        "mla_sparse_chunk": (ctypes.c_int32, [I32, I32]),
        "mla_decode_sparse_kernel_name": (ctypes.c_char_p, [P, I32, I32]),
        "mla_decode_sparse": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, VP, I64, VP, I32, VP,
                                             VP, VP, FP, FP, VP]),
        "mla_draft_positions": (ctypes.c_int, [I32, I32, I32, VP, VP, VP, VP, VP, VP]),
        "mla_index_scores_topk_noalloc": (ctypes.c_int, [P, I32, I32, I32, I32, I32, VP, FP, VP,
                                                         I64, VP, I32, VP, FP, I32, I32, VP, VP,
                                                         VP]),
        "mla_stream_read": (ctypes.c_int, [VP, ctypes.c_size_t, VP, I32, VP]),
        "mla_prefill_workspace_bytes": (ctypes.c_size_t, [P, I32, I32]),
        "mla_prefill_unabsorbed": (ctypes.c_int, [P, I32, I32, VP, VP, VP, VP, VP, I64, VP, I32,
                                                  VP, VP, FP, VP]),
        "mla_prefill_form": (ctypes.c_char_p, [P, I32, I32]),
        "mla_absorb_append_index": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, I32, VP, VP, VP,
                                                   VP, VP, I32, I32, VP, I64, I32, I32, VP, VP,
                                                   VP]),
        "mla_absorb_append_q8": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, I32, VP, VP, VP, VP,
                                                VP, VP, I32, I32, VP, I64, I32, VP]),
        "mla_absorb_append_q4": (ctypes.c_int, [P, I32, VP, VP, VP, VP, VP, I32, VP, VP, VP, VP,
                                                VP, VP, I32, I32, VP, I64, I32, VP]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def status_str(status: int) -> str:
    try:
        return lib().mla_status_str(int(status)).decode()
    except RuntimeError:
        return _STATUS.get(int(status), f"status {status}")


def build_info() -> str:
    return lib().mla_build_info().decode()


def _ck(status: int, where: str):
    if status != 0:
        raise MLAError(status, where)


def config_validate(cfg: Config) -> int:
    return lib().mla_config_validate(cfg.cptr())


def cache_bytes_per_token(cfg: Config) -> int:
    return lib().mla_cache_bytes_per_token(cfg.cptr())


def split_chunk(cfg: Config, seq_len: int, num_splits: int) -> int:
    out = ctypes.c_int32(0)
    _ck(lib().mla_split_chunk(cfg.cptr(), seq_len, num_splits, ctypes.byref(out)),
        "mla_split_chunk")
    return out.value


def default_num_splits(cfg: Config, batch: int, q_len: int, max_seq_len: int,
                       num_cus: int = 256) -> int:
    return lib().mla_default_num_splits(cfg.cptr(), batch, q_len, max_seq_len, num_cus)


def decode_partials_bytes(cfg: Config, batch: int, q_len: int, num_splits: int) -> int:
    return lib().mla_decode_partials_bytes(cfg.cptr(), batch, q_len, num_splits)


def decode_kernel_kind(cfg: Config, q_len: int) -> str:
    """Which decode kernel libmla takes for this shape: "mfma_ws", "mfma_rows16"
    or "generic"."""
    return lib().mla_decode_kernel_name(cfg.cptr(), q_len).decode()


# --------------------------------------------------------------------------
# tensor marshalling
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _elem_dtype(cfg: Config):
    t = _torch()
    return t.float32 if cfg.dtype == F32 else t.bfloat16


def _need(x, name: str, dtype, numel: int):
    t = _torch()
    if not isinstance(x, t.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not x.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if x.dtype != dtype:
        raise TypeError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if x.numel() != numel:
        raise ValueError(f"{name}: {x.numel()} elements, expected {numel}")
    return ctypes.c_void_p(x.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    t = _torch()
    if stream is None:  # the current stream of the current device, as a raw handle
        raw = getattr(t._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return ctypes.c_void_p(raw(t._C._cuda_getDevice()))
        stream = t.cuda.current_stream()
    h = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return ctypes.c_void_p(h)


def _absorb_args(cfg: Config, q_nope, q_rope, pos, w_uk, q_full):
    t = _torch()
    n = int(pos.numel())
    H, dt = cfg.num_heads, _elem_dtype(cfg)
    return (n, _need(q_nope, "q_nope", dt, n * H * cfg.nope_dim),
            _need(q_rope, "q_rope", dt, n * H * cfg.rope_dim),
            _need(pos, "pos", t.int32, n),
            _need(w_uk, "w_uk", dt, H * cfg.nope_dim * cfg.kv_rank),
            _need(q_full, "q_full", dt, n * H * cfg.dim))


def _coded_row(cfg: Config, bits: int) -> int:
    """Bytes per cached row: the workload dtype (bits 0), 8-bit or 4-bit codes."""
    return {0: cfg.dim, 8: cfg.dim + 16, 4: cfg.dim // 2 + 16}[bits]


def _append_args(cfg: Config, c_kv, k_rope, seq_idx, pos, page_table, cache, mode, bits=0):
    t = _torch()
    n = int(pos.numel())
    dt = _elem_dtype(cfg)
    if page_table.dim() != 2:
        raise ValueError("page_table: expected [batch][max_pages]")
    batch, max_pages = page_table.shape
    row = _coded_row(cfg, bits)
    if cache.dim() != 3 or cache.shape[1] != cfg.page_size or cache.shape[2] != row:
        raise ValueError(f"cache: expected [num_pages][{cfg.page_size}][{row}]")
    num_pages = int(cache.shape[0])
    return (n, _need(c_kv, "c_kv", dt, n * cfg.kv_rank),
            _need(k_rope, "k_rope", dt, n * cfg.rope_dim),
            _need(seq_idx, "seq_idx", t.int32, n),
            _need(pos, "pos", t.int32, n),
            _need(page_table, "page_table", t.int32, batch * max_pages),
            int(batch), int(max_pages),
            _need(cache, "cache", t.uint8 if bits else dt, cache.numel()), num_pages, int(mode))


def absorb_q(cfg: Config, q_nope, q_rope, pos, w_uk, q_full, stream=None):
    """a1: q_full[n][h] = [W_UK[h]^T q_nope[n][h] ; RoPE(q_rope[n][h], pos[n])]."""
    args = _absorb_args(cfg, q_nope, q_rope, pos, w_uk, q_full)
    _ck(lib().mla_absorb_q(cfg.cptr(), *args, _stream(stream)), "mla_absorb_q")


def cache_append(cfg: Config, c_kv, k_rope, seq_idx, pos, page_table, cache,
                 mode: int = APPEND_ROTATE, stream=None):
    """a2: write rows [c_kv[n] ; k] at page_table[seq_idx[n]][pos[n] // page] ..."""
    args = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache, mode)
    _ck(lib().mla_cache_append(cfg.cptr(), *args, _stream(stream)), "mla_cache_append")


def absorb_append(cfg: Config, q_nope, q_rope, pos_q, w_uk, q_full, c_kv, k_rope, seq_idx, pos,
                  page_table, cache, mode: int = APPEND_ROTATE, stream=None):
    """a1 + a2 in one launch: absorb_q(q_nope, q_rope, pos_q, w_uk, q_full) and
    cache_append(c_kv, k_rope, seq_idx, pos, page_table, cache, mode)."""
    a = _absorb_args(cfg, q_nope, q_rope, pos_q, w_uk, q_full)
    b = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache, mode)
    _ck(lib().mla_absorb_append(cfg.cptr(), *a, *b, _stream(stream)),
        "mla_absorb_append")


def absorb_append_index(cfg: Config, q_nope, q_rope, pos_q, w_uk, q_full, c_kv, k_rope, seq_idx,
                        pos, page_table, cache, k_idx, index_cache, mode: int = APPEND_ROTATE,
                        stream=None):
    """absorb_append and index_append (the rows' indexer keys k_idx into
    index_cache) in one launch where possible."""
    a = _absorb_args(cfg, q_nope, q_rope, pos_q, w_uk, q_full)
    b = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache, mode)
    n = b[0]
    _, dI = _index_cache_dims(cfg, index_cache)
    dt = _elem_dtype(cfg)
    _ck(lib().mla_absorb_append_index(cfg.cptr(), *a, *b, dI, _need(k_idx, "k_idx", dt, n * dI),
                                      _need(index_cache, "index_cache", dt, index_cache.numel()),
                                      _stream(stream)), "mla_absorb_append_index")


def _rope_pos_arg(rope_pos, n: int):
    if rope_pos is None:
        return None
    return _need(rope_pos, "rope_pos", _torch().int32, n)


def cache_append_at(cfg: Config, c_kv, k_rope, seq_idx, pos, rope_pos, page_table, cache,
                    mode: int = APPEND_ROTATE, stream=None):
    """a2 with row n's RoPE key rotated by rope_pos[n] (None: pos[n]); pos[n]
    still picks the slot (drafted tokens of a tree)."""
    a = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache, mode)
    rp = _rope_pos_arg(rope_pos, a[0])
    _ck(lib().mla_cache_append_at(cfg.cptr(), *a[:5], rp, *a[5:], _stream(stream)),
        "mla_cache_append_at")


def absorb_append_at(cfg: Config, q_nope, q_rope, pos_q, w_uk, q_full, c_kv, k_rope, seq_idx,
                     pos, rope_pos, page_table, cache, mode: int = APPEND_ROTATE, stream=None):
    """absorb_q followed by cache_append_at, in one launch where possible."""
    a = _absorb_args(cfg, q_nope, q_rope, pos_q, w_uk, q_full)
    b = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache, mode)
    rp = _rope_pos_arg(rope_pos, b[0])
    _ck(lib().mla_absorb_append_at(cfg.cptr(), *a, *b[:5], rp, *b[5:],
                                   _stream(stream)), "mla_absorb_append_at")


def draft_positions(seq_lens, q_len: int, max_seq_len: int, tree_parent, seq_idx, slot, pos,
                    stream=None):
    """Drafted-token rows of a verify step, on the device: seq_idx, slot and
    pos [B*Q] int32 (out) from seq_lens [B] and tree_parent [B][Q] (None: a
    chain); -1 slots and positions for an invalid sequence."""
    t = _torch()
    B, Q = int(seq_lens.numel()), int(q_len)
    tp = None if tree_parent is None else _need(tree_parent, "tree_parent", t.int32, B * Q)
    _ck(lib().mla_draft_positions(B, Q, int(max_seq_len), _need(seq_lens, "seq_lens", t.int32, B),
                                  tp, _need(seq_idx, "seq_idx", t.int32, B * Q),
                                  _need(slot, "slot", t.int32, B * Q),
                                  _need(pos, "pos", t.int32, B * Q), _stream(stream)),
        "mla_draft_positions")


def stream_read(buf, sink, stream=None):
    """Read every byte of the device tensor ``buf`` once (16-byte loads);
    sink: a uint32-sized device tensor of one word per block (its numel
    blocks)."""
    t = _torch()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf: must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    blocks = int(sink.numel())
    _ck(lib().mla_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                              _need(sink, "sink", t.int32, blocks), blocks, _stream(stream)),
        "mla_stream_read")


def prefill_workspace_bytes(cfg: Config, seq_len: int, q_len: int) -> int:
    """Bytes of the workspace of prefill_unabsorbed."""
    return int(lib().mla_prefill_workspace_bytes(cfg.cptr(), int(seq_len), int(q_len)))


def prefill_form(cfg: Config, q_len: int, seq_len: int) -> str:
    """"unabsorbed" or "absorbed": the form a prefill chunk should take."""
    return lib().mla_prefill_form(cfg.cptr(), int(q_len), int(seq_len)).decode()


def prefill_unabsorbed(cfg: Config, q_nope, q_rope, w_uk, w_uv, cache, page_row, seq_len: int,
                       workspace, out, lse, stream=None):
    """The unabsorbed prefill of one sequence's newest q_len cached tokens:
    q_nope [q_len][H][d_n], q_rope [q_len][H][d_r] (unrotated), page_row
    [max_pages] int32 (the sequence's page-table row), workspace uint8 of
    prefill_workspace_bytes; out [q_len][H][d_v], lse [q_len][H] f32."""
    t = _torch()
    C = int(q_nope.shape[0])
    H, dt = cfg.num_heads, _elem_dtype(cfg)
    if cache.dim() != 3 or cache.shape[1] != cfg.page_size or cache.shape[2] != cfg.dim:
        raise ValueError(f"cache: expected [num_pages][{cfg.page_size}][{cfg.dim}]")
    max_pages = int(page_row.numel())
    _ck(lib().mla_prefill_unabsorbed(
        cfg.cptr(), C, int(seq_len), _need(q_nope, "q_nope", dt, C * H * cfg.nope_dim),
        _need(q_rope, "q_rope", dt, C * H * cfg.rope_dim),
        _need(w_uk, "w_uk", dt, H * cfg.nope_dim * cfg.kv_rank),
        _need(w_uv, "w_uv", dt, H * cfg.v_dim * cfg.kv_rank),
        _need(cache, "cache", dt, cache.numel()), int(cache.shape[0]),
        _need(page_row, "page_row", t.int32, max_pages), max_pages,
        _need(workspace, "workspace", t.uint8, prefill_workspace_bytes(cfg, seq_len, C)),
        _need(out, "out", dt, C * H * cfg.v_dim), _need(lse, "lse", t.float32, C * H),
        _stream(stream)), "mla_prefill_unabsorbed")


def cache_q8_bytes_per_token(cfg: Config) -> int:
    """Bytes of one 8-bit cache row: d_c + d_r codes + 16 bytes of (min, step)."""
    return lib().mla_cache_q8_bytes_per_token(cfg.cptr())


def cache_append_q8(cfg: Config, c_kv, k_rope, seq_idx, pos, rope_pos, page_table, cache_q8,
                    mode: int = APPEND_ROTATE, stream=None):
    """a2 into an 8-bit cache: cache_q8 uint8 [num_pages][page][D + 16]; each row
    coded per part between its own min and max; rope_pos as cache_append_at."""
    a = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache_q8, mode, bits=8)
    rp = _rope_pos_arg(rope_pos, a[0])
    _ck(lib().mla_cache_append_q8(cfg.cptr(), *a[:5], rp, *a[5:], _stream(stream)),
        "mla_cache_append_q8")


def absorb_append_coded(cfg: Config, bits: int, q_nope, q_rope, pos_q, w_uk, q_full, c_kv,
                        k_rope, seq_idx, pos, rope_pos, page_table, cache,
                        mode: int = APPEND_ROTATE, stream=None):
    """absorb_q followed by cache_append_q8 (bits 8) or cache_append_q4 (bits 4),
    in one launch where possible (mla_absorb_append_q8 / _q4)."""
    if bits not in (8, 4):
        raise ValueError("bits: 8 or 4")
    a = _absorb_args(cfg, q_nope, q_rope, pos_q, w_uk, q_full)
    b = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache, mode, bits=bits)
    rp = _rope_pos_arg(rope_pos, b[0])
    name = "mla_absorb_append_q8" if bits == 8 else "mla_absorb_append_q4"
    _ck(getattr(lib(), name)(cfg.cptr(), *a, *b[:5], rp, *b[5:], _stream(stream)), name)


def cache_q4_bytes_per_token(cfg: Config) -> int:
    """Bytes of one 4-bit cache row: (d_c + d_r) / 2 code bytes + 16 of (min, step)."""
    return lib().mla_cache_q4_bytes_per_token(cfg.cptr())


def cache_append_q4(cfg: Config, c_kv, k_rope, seq_idx, pos, rope_pos, page_table, cache_q4,
                    mode: int = APPEND_ROTATE, stream=None):
    """a2 into a 4-bit cache: cache_q4 uint8 [num_pages][page][D / 2 + 16]; two
    codes per byte (low nibble first); otherwise as cache_append_q8."""
    a = _append_args(cfg, c_kv, k_rope, seq_idx, pos, page_table, cache_q4, mode, bits=4)
    rp = _rope_pos_arg(rope_pos, a[0])
    _ck(lib().mla_cache_append_q4(cfg.cptr(), *a[:5], rp, *a[5:], _stream(stream)),
        "mla_cache_append_q4")


def chunk_plan(cfg: Config, total_tokens: int, max_seq_len: int, num_cus: int = 256):
    """A fixed-size partition plan (chunk_tokens, num_splits) for decode_paged(chunk_tokens=...)."""
    ck, ns = ctypes.c_int32(0), ctypes.c_int32(0)
    _ck(lib().mla_chunk_plan(cfg.cptr(), int(total_tokens), int(max_seq_len),
                             int(num_cus), ctypes.byref(ck), ctypes.byref(ns)), "mla_chunk_plan")
    return ck.value, ns.value


def decode_paged(cfg: Config, q_full, cache, page_table, seq_lens, o_part, lse_part,
                 max_seq_len: int, stream=None, chunk_tokens: int = 0):
    """a4: split-KV partials. q_full [B][Q][H][D]; o_part [B][Q][H][S][d_c] f32;
    lse_part [B][Q][H][S] f32 (S = num_splits from lse_part's last axis).
    chunk_tokens > 0: fixed-size partitions (mla_decode_paged_chunked)."""
    _decode(cfg, q_full, cache, page_table, seq_lens, None, o_part, lse_part, max_seq_len, stream,
            chunk_tokens)


def decode_paged_q8(cfg: Config, q_full, cache_q8, page_table, seq_lens, o_part, lse_part,
                    max_seq_len: int, stream=None, chunk_tokens: int = 0, tree_parent=None):
    """a4 over an 8-bit cache (cache_q8 uint8 [num_pages][page][D + 16]); other
    arguments as decode_paged / decode_paged_tree."""
    _decode(cfg, q_full, cache_q8, page_table, seq_lens, tree_parent, o_part, lse_part,
            max_seq_len, stream, chunk_tokens, bits=8)


def decode_paged_q4(cfg: Config, q_full, cache_q4, page_table, seq_lens, o_part, lse_part,
                    max_seq_len: int, stream=None, chunk_tokens: int = 0, tree_parent=None):
    """a4 over a 4-bit cache (cache_q4 uint8 [num_pages][page][D / 2 + 16]); other
    arguments as decode_paged_q8."""
    _decode(cfg, q_full, cache_q4, page_table, seq_lens, tree_parent, o_part, lse_part,
            max_seq_len, stream, chunk_tokens, bits=4)


def decode_paged_tree(cfg: Config, q_full, cache, page_table, seq_lens, tree_parent, o_part,
                      lse_part, max_seq_len: int, stream=None, chunk_tokens: int = 0):
    """a4 verifying a tree of drafted tokens: tree_parent [B][Q] int32, entry i
    in [-1, i) (the drafted token that token i continues; -1 = the prefix).
    Other arguments as decode_paged."""
    _decode(cfg, q_full, cache, page_table, seq_lens, tree_parent, o_part, lse_part, max_seq_len,
            stream, chunk_tokens)


def _decode(cfg, q_full, cache, page_table, seq_lens, tree_parent, o_part, lse_part, max_seq_len,
            stream, chunk_tokens, bits=0):
    t = _torch()
    if q_full.dim() != 4:
        raise ValueError("q_full: expected [batch][q_len][H][D]")
    B, Q = int(q_full.shape[0]), int(q_full.shape[1])
    if lse_part.dim() != 4:
        raise ValueError("lse_part: expected [batch][q_len][H][num_splits]")
    S = int(lse_part.shape[3])
    H, dt = cfg.num_heads, _elem_dtype(cfg)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table: expected [batch][max_pages]")
    max_pages = int(page_table.shape[1])
    row = _coded_row(cfg, bits)
    if cache.dim() != 3 or cache.shape[1] != cfg.page_size or cache.shape[2] != row:
        raise ValueError(f"cache: expected [num_pages][{cfg.page_size}][{row}]")
    num_pages = int(cache.shape[0])
    args = (_need(q_full, "q_full", dt, B * Q * H * cfg.dim),
            _need(cache, "cache", t.uint8 if bits else dt, cache.numel()))
    pt = _need(page_table, "page_table", t.int32, B * max_pages)
    sl = _need(seq_lens, "seq_lens", t.int32, B)
    op = _need(o_part, "o_part", t.float32, B * Q * H * S * cfg.kv_rank)
    lp = _need(lse_part, "lse_part", t.float32, B * Q * H * S)
    if bits:
        tp = None if tree_parent is None else _need(tree_parent, "tree_parent", t.int32, B * Q)
        name = "mla_decode_paged_q8" if bits == 8 else "mla_decode_paged_q4"
        _ck(getattr(lib(), name)(cfg.cptr(), B, Q, int(chunk_tokens), S, int(max_seq_len),
                                 args[0], args[1], num_pages, pt, max_pages, sl, tp, op, lp,
                                 _stream(stream)), name)
        return
    if tree_parent is not None:
        tp = _need(tree_parent, "tree_parent", t.int32, B * Q)
        _ck(lib().mla_decode_paged_tree(cfg.cptr(), B, Q, int(chunk_tokens), S,
                                        int(max_seq_len), args[0], args[1], num_pages, pt,
                                        max_pages, sl, tp, op, lp, _stream(stream)),
            "mla_decode_paged_tree")
        return
    if chunk_tokens:
        _ck(lib().mla_decode_paged_chunked(cfg.cptr(), B, Q, int(chunk_tokens), S,
                                           int(max_seq_len), args[0], args[1], num_pages, pt,
                                           max_pages, sl, op, lp, _stream(stream)),
            "mla_decode_paged_chunked")
        return
    _ck(lib().mla_decode_paged(cfg.cptr(), B, Q, S, int(max_seq_len), args[0], args[1],
                               num_pages, pt, max_pages, sl, op, lp, _stream(stream)),
        "mla_decode_paged")


# --------------------------------------------------------------------------
# sparse read
# --------------------------------------------------------------------------
def _index_cache_dims(cfg: Config, index_cache):
    if index_cache.dim() != 3 or index_cache.shape[1] != cfg.page_size:
        raise ValueError(f"index_cache: expected [num_pages][{cfg.page_size}][index_dim]")
    return int(index_cache.shape[0]), int(index_cache.shape[2])


def index_append(cfg: Config, k_idx, seq_idx, pos, page_table, index_cache, stream=None):
    """Indexer keys k_idx [n][index_dim] into index_cache [num_pages][page][index_dim]
    at the slots mla_cache_append would pick (no rotation)."""
    t = _torch()
    n = int(pos.numel())
    num_pages, dI = _index_cache_dims(cfg, index_cache)
    if page_table.dim() != 2:
        raise ValueError("page_table: expected [batch][max_pages]")
    batch, max_pages = (int(x) for x in page_table.shape)
    dt = _elem_dtype(cfg)
    _ck(lib().mla_index_append(cfg.cptr(), dI, n, _need(k_idx, "k_idx", dt, n * dI),
                               _need(seq_idx, "seq_idx", t.int32, n), _need(pos, "pos", t.int32, n),
                               _need(page_table, "page_table", t.int32, batch * max_pages), batch,
                               max_pages, _need(index_cache, "index_cache", dt, index_cache.numel()),
                               num_pages, _stream(stream)), "mla_index_append")


def index_scores(cfg: Config, q_idx, w_idx, index_cache, page_table, seq_lens, scores,
                 max_seq_len: int, stream=None):
    """Index scores [B][Q][ld] f32 (ld = scores.shape[2] >= max_seq_len):
    sum_h w_idx[b][j][h] * max(0, q_idx[b][j][h] . k_idx(b, t)) for t < L_b.
    q_idx [B][Q][H_I][d_I] (cfg dtype), w_idx [B][Q][H_I] f32."""
    t = _torch()
    if q_idx.dim() != 4 or scores.dim() != 3:
        raise ValueError("q_idx: expected [batch][q_len][heads][dim]; scores [batch][q_len][ld]")
    B, Q, Hi, dI = (int(x) for x in q_idx.shape)
    num_pages, dI2 = _index_cache_dims(cfg, index_cache)
    if dI2 != dI:
        raise ValueError("index_cache width does not match q_idx")
    max_pages = int(page_table.shape[1])
    ld = int(scores.shape[2])
    dt = _elem_dtype(cfg)
    _ck(lib().mla_index_scores(cfg.cptr(), Hi, dI, B, Q, int(max_seq_len),
                               _need(q_idx, "q_idx", dt, B * Q * Hi * dI),
                               _need(w_idx, "w_idx", t.float32, B * Q * Hi),
                               _need(index_cache, "index_cache", dt, index_cache.numel()),
                               num_pages, _need(page_table, "page_table", t.int32, B * max_pages),
                               max_pages, _need(seq_lens, "seq_lens", t.int32, B),
                               _need(scores, "scores", t.float32, B * Q * ld), ld,
                               _stream(stream)), "mla_index_scores")


def index_scores_topk(cfg: Config, q_idx, w_idx, index_cache, page_table, seq_lens, scores,
                      max_seq_len: int, indices, counts, workspace, stream=None):
    """index_scores then topk_select in one library call (the same scores,
    indices and counts; one launch fewer with the MFMA indexer)."""
    t = _torch()
    if q_idx.dim() != 4 or scores.dim() != 3 or indices.dim() != 3:
        raise ValueError("q_idx: expected [batch][q_len][heads][dim]; scores [batch][q_len][ld]; "
                         "indices [batch][q_len][topk]")
    B, Q, Hi, dI = (int(x) for x in q_idx.shape)
    num_pages, dI2 = _index_cache_dims(cfg, index_cache)
    if dI2 != dI:
        raise ValueError("index_cache width does not match q_idx")
    max_pages = int(page_table.shape[1])
    ld = int(scores.shape[2])
    K = int(indices.shape[2])
    dt = _elem_dtype(cfg)
    _ck(lib().mla_index_scores_topk(cfg.cptr(), Hi, dI, B, Q, int(max_seq_len),
                                    _need(q_idx, "q_idx", dt, B * Q * Hi * dI),
                                    _need(w_idx, "w_idx", t.float32, B * Q * Hi),
                                    _need(index_cache, "index_cache", dt, index_cache.numel()),
                                    num_pages,
                                    _need(page_table, "page_table", t.int32, B * max_pages),
                                    max_pages, _need(seq_lens, "seq_lens", t.int32, B),
                                    _need(scores, "scores", t.float32, B * Q * ld), ld, K,
                                    _need(workspace, "workspace", t.uint8,
                                          topk_workspace_bytes(B, Q)),
                                    _need(indices, "indices", t.int32, B * Q * K),
                                    _need(counts, "counts", t.int32, B * Q), _stream(stream)),
        "mla_index_scores_topk")


TOPK_NOALLOC_MAX_QUERIES = 256  # MLA_TOPK_NOALLOC_MAX_QUERIES


def index_scores_topk_noalloc(cfg: Config, q_idx, w_idx, index_cache, page_table, seq_lens,
                              scores, max_seq_len: int, indices, counts, stream=None):
    """index_scores_topk with the workspace held inside the library (no
    device allocation by the call; batch * q_len <= TOPK_NOALLOC_MAX_QUERIES).
    Calls that overlap on one GPU race on that workspace."""
    t = _torch()
    if q_idx.dim() != 4 or scores.dim() != 3 or indices.dim() != 3:
        raise ValueError("q_idx: expected [batch][q_len][heads][dim]; scores [batch][q_len][ld]; "
                         "indices [batch][q_len][topk]")
    B, Q, Hi, dI = (int(x) for x in q_idx.shape)
    num_pages, dI2 = _index_cache_dims(cfg, index_cache)
    if dI2 != dI:
        raise ValueError("index_cache width does not match q_idx")
    max_pages = int(page_table.shape[1])
    ld = int(scores.shape[2])
    K = int(indices.shape[2])
    dt = _elem_dtype(cfg)
    _ck(lib().mla_index_scores_topk_noalloc(
        cfg.cptr(), Hi, dI, B, Q, int(max_seq_len), _need(q_idx, "q_idx", dt, B * Q * Hi * dI),
        _need(w_idx, "w_idx", t.float32, B * Q * Hi),
        _need(index_cache, "index_cache", dt, index_cache.numel()), num_pages,
        _need(page_table, "page_table", t.int32, B * max_pages), max_pages,
        _need(seq_lens, "seq_lens", t.int32, B), _need(scores, "scores", t.float32, B * Q * ld),
        ld, K, _need(indices, "indices", t.int32, B * Q * K),
        _need(counts, "counts", t.int32, B * Q), _stream(stream)),
        "mla_index_scores_topk_noalloc")


def topk_workspace_bytes(batch: int, q_len: int) -> int:
    """Bytes of the top-k workspace (allocate zeroed once; every call leaves it zero)."""
    return int(lib().mla_topk_workspace_bytes(int(batch), int(q_len)))


def topk_select(scores, seq_lens, indices, counts, max_seq_len: int, workspace, stream=None):
    """The topk (= indices.shape[2]) best-scored tokens each query sees, in
    increasing token order; counts [B][Q] int32 (-1: invalid sequence).
    workspace: a uint8 device tensor of topk_workspace_bytes(B, Q), zero on
    the first call (the call leaves it zero)."""
    t = _torch()
    if scores.dim() != 3 or indices.dim() != 3:
        raise ValueError("scores: expected [batch][q_len][ld]; indices [batch][q_len][topk]")
    B, Q, ld = (int(x) for x in scores.shape)
    K = int(indices.shape[2])
    _ck(lib().mla_topk_select(B, Q, int(max_seq_len), K,
                              _need(scores, "scores", t.float32, B * Q * ld), ld,
                              _need(seq_lens, "seq_lens", t.int32, B),
                              _need(workspace, "workspace", t.uint8, topk_workspace_bytes(B, Q)),
                              _need(indices, "indices", t.int32, B * Q * K),
                              _need(counts, "counts", t.int32, B * Q), _stream(stream)),
        "mla_topk_select")


def sparse_chunk(topk: int, num_splits: int) -> int:
    """List entries per partition of decode_sparse."""
    return int(lib().mla_sparse_chunk(int(topk), int(num_splits)))


def decode_sparse_kernel_kind(cfg: Config, topk: int, num_splits: int) -> str:
    """"mfma_rows16_gather" or "generic_gather"."""
    return lib().mla_decode_sparse_kernel_name(cfg.cptr(), int(topk),
                                               int(num_splits)).decode()


def decode_sparse(cfg: Config, q_full, cache, page_table, seq_lens, indices, counts, o_part,
                  lse_part, max_seq_len: int, stream=None):
    """a4 over the selected tokens indices [B][Q][topk] (counts [B][Q]); other
    arguments and outputs as decode_paged."""
    t = _torch()
    B, Q = int(q_full.shape[0]), int(q_full.shape[1])
    S = int(lse_part.shape[3])
    K = int(indices.shape[2])
    H, dt = cfg.num_heads, _elem_dtype(cfg)
    if cache.dim() != 3 or cache.shape[1] != cfg.page_size or cache.shape[2] != cfg.dim:
        raise ValueError(f"cache: expected [num_pages][{cfg.page_size}][{cfg.dim}]")
    max_pages = int(page_table.shape[1])
    _ck(lib().mla_decode_sparse(cfg.cptr(), B, Q, K, S, int(max_seq_len),
                                _need(q_full, "q_full", dt, B * Q * H * cfg.dim),
                                _need(cache, "cache", dt, cache.numel()), int(cache.shape[0]),
                                _need(page_table, "page_table", t.int32, B * max_pages), max_pages,
                                _need(seq_lens, "seq_lens", t.int32, B),
                                _need(indices, "indices", t.int32, B * Q * K),
                                _need(counts, "counts", t.int32, B * Q),
                                _need(o_part, "o_part", t.float32, B * Q * H * S * cfg.kv_rank),
                                _need(lse_part, "lse_part", t.float32, B * Q * H * S),
                                _stream(stream)), "mla_decode_sparse")


def _combine_args(cfg: Config, o_part, lse_part, o_lat, lse):
    t = _torch()
    if lse_part.dim() != 4:
        raise ValueError("lse_part: expected [batch][q_len][H][num_splits]")
    B, Q, H, S = (int(x) for x in lse_part.shape)
    if H != cfg.num_heads:
        raise ValueError("lse_part: head axis does not match cfg.num_heads")
    dt = _elem_dtype(cfg)
    op = _need(o_part, "o_part", t.float32, B * Q * H * S * cfg.kv_rank)
    lp = _need(lse_part, "lse_part", t.float32, B * Q * H * S)
    ol = _need(o_lat, "o_lat", dt, B * Q * H * cfg.kv_rank)
    ls = ctypes.c_void_p(None) if lse is None else _need(lse, "lse", t.float32, B * Q * H)
    return (B, Q, S, op, lp, ol, ls)


def splitkv_combine(cfg: Config, o_part, lse_part, o_lat, lse=None, stream=None):
    """a5: LSE merge. o_lat [B][Q][H][d_c] (cfg dtype); lse [B][Q][H] f32 or None."""
    args = _combine_args(cfg, o_part, lse_part, o_lat, lse)
    _ck(lib().mla_splitkv_combine(cfg.cptr(), *args, _stream(stream)),
        "mla_splitkv_combine")


def combine_up_project(cfg: Config, o_part, lse_part, o_lat, w_uv, out, lse=None, stream=None):
    """a5 + a6 in one launch: splitkv_combine(o_part, lse_part, o_lat, lse), then
    up_project_v(o_lat, w_uv, out); out [B][Q][H][d_v]."""
    B, Q, S, op, lp, ol, ls = _combine_args(cfg, o_part, lse_part, o_lat, lse)
    H, dt = cfg.num_heads, _elem_dtype(cfg)
    wv = _need(w_uv, "w_uv", dt, H * cfg.v_dim * cfg.kv_rank)
    ot = _need(out, "out", dt, B * Q * H * cfg.v_dim)
    _ck(lib().mla_combine_up_project(cfg.cptr(), B, Q, S, op, lp, ol, ls, wv, ot,
                                     _stream(stream)), "mla_combine_up_project")


def up_project_v(cfg: Config, o_lat, w_uv, out, stream=None):
    """a6: out[n][h] = W_UV[h] o_lat[n][h]; o_lat [N][H][d_c] -> out [N][H][d_v]."""
    H, dt = cfg.num_heads, _elem_dtype(cfg)
    n = int(o_lat.numel()) // (H * cfg.kv_rank)
    args = (_need(o_lat, "o_lat", dt, n * H * cfg.kv_rank),
            _need(w_uv, "w_uv", dt, H * cfg.v_dim * cfg.kv_rank),
            _need(out, "out", dt, n * H * cfg.v_dim))
    _ck(lib().mla_up_project_v(cfg.cptr(), n, *args, _stream(stream)), "mla_up_project_v")
